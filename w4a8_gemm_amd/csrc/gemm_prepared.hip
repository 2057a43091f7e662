// gemm_prepared.hip -- MXFP4 weights in matrix-core fragment order, and the
// decode GEMM that streams them.
//
// "vllm-radiance (MXFP4)", How the MXFP4 path works: the W4A8 kernel streams
// weights repacked at load time into the order its matrix instructions consume
// (there for gfx1201 WMMA fragments).  This is the CDNA4 equivalent for
// V_MFMA_SCALE_F32_16X16X128_F8F6F4 with the weight as the e2m1 A operand:
//
//   weight blocks  one 1 KiB block per (16-row tile t, 128-wide K step s), blocks
//                  ordered t-major; inside a block lane L = n + 16g (n < 16,
//                  g < 4) owns 16 bytes = row 16t + n, packed bytes
//                  [64s + 16g, 64s + 16g + 16) (k = 128s + 32g .. +31).
//   scale dwords   one 256-byte block per (tile t, 4-step chunk c); lane L owns
//                  a dword whose byte u is the e8m0 of row 16t + n, K-block
//                  4(4c + u) + g, so MFMA u of the chunk takes it with opsel u.
//   padding        steps are padded to a multiple of 4 and rows to a multiple
//                  of 16 with zero codes and e8m0 127 (1.0).
//
// A wavefront then reads every weight and scale byte in whole contiguous
// 1 KiB / 256 B runs, exactly once, and nothing needs rearranging in registers.
#include <type_traits>

#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kFmtFp8 = 0;
constexpr int kFmtFp4 = 4;
constexpr int kUnitScale = 127;

__device__ __forceinline__ v8i frag_fp4(uint4 q) {
    v8i r = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
    return r;
}
__device__ __forceinline__ v8i frag_fp8(uint4 lo, uint4 hi) {
    v8i r = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    return r;
}
template <int OPSEL>
__device__ __forceinline__ v4f mfma16(v8i a_fp4, v8i b_fp8, v4f c, int scale_a) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_fp4, b_fp8, c, kFmtFp4, kFmtFp8, OPSEL,
                                                            scale_a, 0, kUnitScale);
}
// fp4 x fp4: weight scale byte OPSEL of scale_a, activation scale in the low
// byte of scale_b
template <int OPSEL>
__device__ __forceinline__ v4f mfma44(v8i a_fp4, v8i b_fp4, v4f c, int scale_a, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_fp4, b_fp4, c, kFmtFp4, kFmtFp4, OPSEL, scale_a,
                                                            0, scale_b);
}

// Weight formats of the fragment-order layout (same 1 KiB block per 16-row
// tile and 128-wide K step, same lane order; the activation operand is the
// same for both):
//   kWMx  MXFP4: e2m1 codes (lane bytes = k 32g .. 32g+31), e8m0 scales as a
//         dword per lane and 4-step chunk, applied by the MFMA's scale operand.
//   kWI4  symmetric int4 g128: codes c (value c - 8) in the same nibble order
//         (lane bytes = k 32g .. 32g+31, low nibble even k); one fp16 scale
//         per weight row and step, applied to the step's products in fp32.
//         The tiled kernels widen the codes to e4m3 in registers and multiply
//         fp8 x fp8, the activation fragment read in the same k order (the
//         dot product is indifferent to how k is dealt to the operand bytes,
//         as long as both operands agree).  The split-K decode kernels, where
//         each weight fragment meets one or a few activation fragments and
//         the widening would bound the kernel, split the code instead:
//         c - 8 = 2 (c & 3)/2 + 8 ((c >> 2) & 3)/2 - 8, two e2m1 fragments
//         (codes 0..3 are the values 0, 0.5, 1, 1.5) taken with one mask each,
//         scaled by 2 and 8 through the matrix core's e8m0 operand, and the
//         -8 sum(x) term from a constant fragment (-1 x 8) fed in as the
//         accumulator input.
//   kWMxA4  MXFP4 weights as kWMx, multiplied with MXFP4 activations (e2m1
//         codes and an e8m0 scale per 32 k of a token) on the fp4 x fp4
//         product; only the split-K decode kernel takes it (the tiled W4A4
//         kernel is its own).
//   kWI4Z int4 g128 with a zero point z per group and row: the codes as kWI4.
//         The decode kernels take products against c - 8 as there and add
//         (8 - z) x (the group's activation sum) per group before its row
//         scale, the sum from the constant fragment's -8 sum(x).  The tiled
//         kernels widen c - z directly (exact in e4m3: -16..14), each lane
//         through the 16-byte table of its row's z, read from a 16-table LDS
//         block.  Scales and zeros share one 256-byte record per 16-row tile
//         and 4-step chunk: fp16 scales, then bytes 16 - z, then padding,
//         scales and bytes in lane-group order [row / 4][step][row % 4]
//         (a decode lane reads its chunk's scales as 32 contiguous bytes
//         and its zero bytes as 16).
//   kWI5  int5 g128: the low four bits of each code as kWI4's nibbles, the
//         fifth bits in a plane of one word per lane and step whose bit
//         8 q + 2 i + p is the fifth bit of the lane's code 8 i + 2 q + p
//         (the checkpoint word with its 2-bit units transposed as a 4 x 4
//         array, so that each byte's bits for even and odd codes sit in
//         one column), stored [tile][chunk][lane][step] so that a lane
//         reads a chunk's four words with one load.  The split-K decode kernel takes c - 16 = 2 v(c & 3) +
//         8 v((c >> 2) & 3) + 16 b4 - 16 as four fp4 x fp8 products (the
//         fifth bits spread to e2m1 1.0 nibbles, scale 16) and folds
//         (16 - z) x sum(x) per step.  The tiled kernel widens c - 16 to e4m3
//         (exact: -16..15) through four 8-byte tables, and adds the
//         zero-point term sum over a chunk's four steps of
//         s (16 - z) x sum(x) with one fp32 16x16x4 product per output
//         tile, the token-and-group activation sums from a pre-pass.
//         Records as kWI4Z with the bytes 16 - z (signed).
constexpr int kWMx = 0, kWI4 = 1, kWMxA4 = 2, kWI4Z = 3, kWI5 = 4;
template <int WF> constexpr bool kIsI4 = WF == kWI4 || WF == kWI4Z;
// formats the tiled kernel widens to e4m3 in registers (one wave row)
template <int WF> constexpr bool kWiden = kIsI4<WF> || WF == kWI5;

template <int WF> struct WStep;                               // per-step scale data of a lane
template <> struct WStep<kWMx> { using T = uint32_t; };      // e8m0 dword (byte = step % 4)
template <> struct WStep<kWI4> { using T = uint2; };         // fp16 scales of its 4 output rows
template <> struct WStep<kWMxA4> { using T = uint32_t; };
template <> struct WStep<kWI4Z> { using T = uint2; };
template <> struct WStep<kWI5> { using T = uint2; };

// a lane's activation fragment (B operand) from its LDS row (16-byte chunks
// XOR-swizzled by sw): MXFP4 pairs with the fp8 operand's own k order, the
// widened int4 codes with 32 consecutive k
template <int WF>
__device__ __forceinline__ v8i act_frag(const uint8_t* rowp, int g, int sw) {
    const int c0 = WF == kWMx ? g : 2 * g, c1 = WF == kWMx ? 4 + g : 2 * g + 1;
    return frag_fp8(*reinterpret_cast<const uint4*>(rowp + 16 * (c0 ^ sw)),
                    *reinterpret_cast<const uint4*>(rowp + 16 * (c1 ^ sw)));
}

// a lane's weight fragment (A operand) from its 16 stored bytes
template <int WF>
__device__ __forceinline__ v8i wfrag(uint4 q) {
    if constexpr (WF == kWMx) {
        return frag_fp4(q);
    } else {
        const uint2 a = int4x8_to_e4m3(q.x), b = int4x8_to_e4m3(q.y);
        const uint2 c = int4x8_to_e4m3(q.z), d = int4x8_to_e4m3(q.w);
        v8i r = {(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y, (int)d.x, (int)d.y};
        return r;
    }
}

// acc += one K step's products (MXFP4: e8m0 byte OPSEL of the dword)
template <int WF, int OPSEL>
__device__ __forceinline__ v4f wmma(v8i a, v8i b, v4f acc, typename WStep<WF>::T sc) {
    if constexpr (WF == kWMx) {
        return mfma16<OPSEL>(a, b, acc, (int)sc);
    } else {
        const v4f t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, v4f{0.f, 0.f, 0.f, 0.f}, kFmtFp8,
                                                                       kFmtFp8, 0, kUnitScale, 0, kUnitScale);
        acc[0] = __builtin_fmaf(f16_to_f32(sc.x & 0xFFFFu), t[0], acc[0]);
        acc[1] = __builtin_fmaf(f16_to_f32(sc.x >> 16), t[1], acc[1]);
        acc[2] = __builtin_fmaf(f16_to_f32(sc.y & 0xFFFFu), t[2], acc[2]);
        acc[3] = __builtin_fmaf(f16_to_f32(sc.y >> 16), t[3], acc[3]);
        return acc;
    }
}

// Decode kernels, int4: the two e2m1 halves of a lane's 16 stored bytes
struct I4Split {
    v8i lo, hi;
};
__device__ __forceinline__ I4Split i4_split(uint4 q) {
    constexpr uint32_t m = 0x33333333u;
    I4Split r;
    r.lo = frag_fp4(make_uint4(q.x & m, q.y & m, q.z & m, q.w & m));
    r.hi = frag_fp4(make_uint4((q.x >> 2) & m, (q.y >> 2) & m, (q.z >> 2) & m, (q.w >> 2) & m));
    return r;
}
// acc += scale(row) * (x . (c - 8)) over one K step
__device__ __forceinline__ v4f i4_split_mma(const I4Split& w, v8i bx, v4f acc, uint2 sc) {
    constexpr int kX2 = 128, kX8 = 130;                       // e8m0 2^1, 2^3
    const v8i neg1 = {(int)0xAAAAAAAA, (int)0xAAAAAAAA, (int)0xAAAAAAAA, (int)0xAAAAAAAA, 0, 0, 0, 0};
    v4f t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(neg1, bx, v4f{0.f, 0.f, 0.f, 0.f}, kFmtFp4,
                                                             kFmtFp8, 0, kX8, 0, kUnitScale);
    t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.lo, bx, t, kFmtFp4, kFmtFp8, 0, kX2, 0, kUnitScale);
    t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.hi, bx, t, kFmtFp4, kFmtFp8, 0, kX8, 0, kUnitScale);
    acc[0] = __builtin_fmaf(f16_to_f32(sc.x & 0xFFFFu), t[0], acc[0]);
    acc[1] = __builtin_fmaf(f16_to_f32(sc.x >> 16), t[1], acc[1]);
    acc[2] = __builtin_fmaf(f16_to_f32(sc.y & 0xFFFFu), t[2], acc[2]);
    acc[3] = __builtin_fmaf(f16_to_f32(sc.y >> 16), t[3], acc[3]);
    return acc;
}

// the same with a zero point per row: acc += scale(row) * (x . (c - z)), from
// x . (c - 8) and (8 - z) * sum(x), sum(x) = -t0 / 8 of the constant product;
// zb: bytes 16 - z of the lane's four rows
__device__ __forceinline__ v4f i4z_split_mma(const I4Split& w, v8i bx, v4f acc, uint2 sc, uint32_t zb) {
    constexpr int kX2 = 128, kX8 = 130;
    const v8i neg1 = {(int)0xAAAAAAAA, (int)0xAAAAAAAA, (int)0xAAAAAAAA, (int)0xAAAAAAAA, 0, 0, 0, 0};
    const v4f t0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(neg1, bx, v4f{0.f, 0.f, 0.f, 0.f}, kFmtFp4,
                                                                    kFmtFp8, 0, kX8, 0, kUnitScale);
    v4f t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.lo, bx, t0, kFmtFp4, kFmtFp8, 0, kX2, 0, kUnitScale);
    t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.hi, bx, t, kFmtFp4, kFmtFp8, 0, kX8, 0, kUnitScale);
    const float s4[4] = {f16_to_f32(sc.x & 0xFFFFu), f16_to_f32(sc.x >> 16), f16_to_f32(sc.y & 0xFFFFu),
                         f16_to_f32(sc.y >> 16)};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float zo = (float)((int)((zb >> (8 * r)) & 0xFFu) - 8);     // 8 - z
        const float u = __builtin_fmaf(zo * -0.125f, t0[r], t[r]);
        acc[r] = __builtin_fmaf(s4[r], u, acc[r]);
    }
    return acc;
}

// int5: the fifth bits of a lane's 32 codes (bit j = k 32g + j) as an e2m1
// fragment, nibble j = 2 (value 1.0) where the bit is set
__device__ __forceinline__ v8i i5_bit_frag(uint32_t b) {
    // plane bit 8 q + 2 i + p is the fifth bit of code 8 i + 2 q + p: word i's
    // byte q takes bits p = 0, 1 of (b >> 2 i) into the low and high nibble
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = b >> (2 * i);
        w[i] = ((x << 1) & 0x02020202u) | ((x << 4) & 0x20202020u);
    }
    return v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
}
// acc += scale(row) * (x . (c - z)) over one K step for int5 codes: x . (c - 16)
// from four products, then (16 - z) * sum(x), sum(x) = -t0 / 16; zb: signed
// bytes 16 - z of the lane's four rows
__device__ __forceinline__ v4f i5_split_mma(const I4Split& w, v8i b4, v8i bx, v4f acc, uint2 sc, uint32_t zb) {
    constexpr int kX2 = 128, kX8 = 130, kX16 = 131;
    const v8i neg1 = {(int)0xAAAAAAAA, (int)0xAAAAAAAA, (int)0xAAAAAAAA, (int)0xAAAAAAAA, 0, 0, 0, 0};
    const v4f t0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(neg1, bx, v4f{0.f, 0.f, 0.f, 0.f}, kFmtFp4,
                                                                    kFmtFp8, 0, kX16, 0, kUnitScale);
    v4f t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.lo, bx, t0, kFmtFp4, kFmtFp8, 0, kX2, 0, kUnitScale);
    t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.hi, bx, t, kFmtFp4, kFmtFp8, 0, kX8, 0, kUnitScale);
    t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b4, bx, t, kFmtFp4, kFmtFp8, 0, kX16, 0, kUnitScale);
    const float s4[4] = {f16_to_f32(sc.x & 0xFFFFu), f16_to_f32(sc.x >> 16), f16_to_f32(sc.y & 0xFFFFu),
                         f16_to_f32(sc.y >> 16)};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float zo = (float)(int)(int8_t)((zb >> (8 * r)) & 0xFFu);    // 16 - z
        const float u = __builtin_fmaf(zo * -0.0625f, t0[r], t[r]);
        acc[r] = __builtin_fmaf(s4[r], u, acc[r]);
    }
    return acc;
}

// ---------------------------------------------------------------------------
// prepare: plain [N, K/2] codes + [N, K/32] e8m0 -> fragment order
// ---------------------------------------------------------------------------

// (also the int4 [N, K/8] layout, whose row n holds the same 16-byte lane
// items at the same offsets: padding then the int4 zero code 8 in every nibble)
__global__ __launch_bounds__(256) void prep_w_kernel(const uint8_t* __restrict__ wq, int N, int K,
                                                     int tiles, int s_pad, uint4* __restrict__ wt,
                                                     uint32_t pad) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)tiles * s_pad * 64) return;
    const int L = (int)(i & 63);
    const int64_t blk = i >> 6;
    const int s = (int)(blk % s_pad), t = (int)(blk / s_pad);
    const int row = 16 * t + (L & 15), g = L >> 4;
    uint4 v = make_uint4(pad, pad, pad, pad);
    if (row < N && s < K / 128)
        v = *reinterpret_cast<const uint4*>(wq + (int64_t)row * (K / 2) + 64 * (int64_t)s + 16 * g);
    wt[i] = v;
}

__global__ __launch_bounds__(256) void prep_s_kernel(const uint8_t* __restrict__ we, int N, int K,
                                                     int tiles, int c_pad, uint32_t* __restrict__ st) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)tiles * c_pad * 64) return;
    const int L = (int)(i & 63);
    const int64_t blk = i >> 6;
    const int c = (int)(blk % c_pad), t = (int)(blk / c_pad);
    const int row = 16 * t + (L & 15), g = L >> 4;
    const int steps = K / 128;
    uint32_t d = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int s = 4 * c + u;
        const uint32_t b = (row < N && s < steps) ? we[(int64_t)row * (K / 32) + 4 * s + g] : (uint32_t)kUnitScale;
        d |= b << (8 * u);
    }
    st[i] = d;
}

// int4 g128 -> fragment order.  Weights from the checkpoint layout qweight
// [K/8, N] (nibble j of word i is k = 8i + j): block (t, s), lane L = n + 16g
// takes words 16s + 4g .. 16s + 4g + 3 (k = 128s + 32g .. +31) of column
// 16t + n -- the MXFP4 layout's k order.  Padding rows and steps hold code 8
// (value 0).  Scales [K/128, N] fp16 -> [tile][chunk][step][16 rows], padding 0.
__global__ __launch_bounds__(256) void prep_i4w_kernel(const uint32_t* __restrict__ qkn, int N, int K,
                                                       int tiles, int s_pad, uint4* __restrict__ wt) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)tiles * s_pad * 64) return;
    const int L = (int)(i & 63);
    const int64_t blk = i >> 6;
    const int s = (int)(blk % s_pad), t = (int)(blk / s_pad);
    const int row = 16 * t + (L & 15), g = L >> 4;
    uint4 v = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
    if (row < N && s < K / 128) {
        const int64_t i0 = 16 * (int64_t)s + 4 * g;
        v.x = qkn[i0 * N + row];
        v.y = qkn[(i0 + 1) * N + row];
        v.z = qkn[(i0 + 2) * N + row];
        v.w = qkn[(i0 + 3) * N + row];
    }
    wt[i] = v;
}

__global__ __launch_bounds__(256) void prep_i4s_kernel(const uint16_t* __restrict__ sc, int N, int K,
                                                       int tiles, int c_pad, uint16_t* __restrict__ st) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)tiles * c_pad * 64) return;
    const int r = (int)(i & 15);
    const int u = (int)((i >> 4) & 3);
    const int64_t tc = i >> 6;
    const int c = (int)(tc % c_pad), t = (int)(tc / c_pad);
    const int s = 4 * c + u, n = 16 * t + r;
    // lane-group order: rows 4q .. 4q + 3 of all four steps in 32 bytes
    st[tc * 64 + 16 * (r >> 2) + 4 * u + (r & 3)] = (n < N && s < K / 128) ? sc[(int64_t)s * N + n] : (uint16_t)0;
}

// int4 with zero points: one 256-byte record per (16-row tile, 4-step chunk):
// fp16 scales (bytes 0..127), bytes 16 - z (128..191; z - 1 is nibble n % 8
// of qzeros[s, n / 8]), zero padding (192..255); scales and bytes in
// lane-group order [row / 4][step][row % 4], so that the 16 lanes that share
// four output rows read their chunk's scales as 32 contiguous bytes and
// their zero bytes as 16.  Rows
// past N and steps past K get scale 0 and z = 8.  One thread per (record, step,
// row), the first 64 also clearing the padding.
__global__ __launch_bounds__(256) void prep_i4zs_kernel(const uint16_t* __restrict__ sc,
                                                        const uint32_t* __restrict__ qz, int N, int K, int tiles,
                                                        int c_pad, uint8_t* __restrict__ st) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)tiles * c_pad * 64) return;
    const int r = (int)(i & 15);
    const int u = (int)((i >> 4) & 3);
    const int64_t tc = i >> 6;
    const int c = (int)(tc % c_pad), t = (int)(tc / c_pad);
    const int s = 4 * c + u, n = 16 * t + r;
    const bool in = n < N && s < K / 128;
    uint8_t* rec = st + 256 * tc;
    const int e = 16 * (r >> 2) + 4 * u + (r & 3);
    reinterpret_cast<uint16_t*>(rec)[e] = in ? sc[(int64_t)s * N + n] : (uint16_t)0;
    rec[128 + e] = in ? (uint8_t)(15u - ((qz[(int64_t)s * (N / 8) + n / 8] >> (4 * (n % 8))) & 15u)) : (uint8_t)8;
    rec[192 + e] = 0;
}

// int5: the fifth-bit plane, one word per (tile, chunk, lane, step): lane L's 32
// codes (row 16t + L % 16, k = 128s + 32(L / 16) + j) are bits j of the
// checkpoint word qweight_hi[4s + L / 16, row]; zero past N or K
__global__ __launch_bounds__(256) void prep_i5b_kernel(const uint32_t* __restrict__ qhi, int N, int K, int tiles,
                                                       int s_pad, uint32_t* __restrict__ w5) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)tiles * s_pad * 64) return;
    const int L = (int)(i & 63);
    const int64_t blk = i >> 6;
    const int s = (int)(blk % s_pad), t = (int)(blk / s_pad);
    const int row = 16 * t + (L & 15), g = L >> 4;
    const uint32_t h = (row < N && s < K / 128) ? qhi[(int64_t)(4 * s + g) * N + row] : 0u;
    // bit pair (8 i + 2 q, +1) of the checkpoint word -> bits 8 q + 2 i, +1
    uint32_t o = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) o |= ((h >> (8 * (u >> 2) + 2 * (u & 3))) & 3u) << (8 * (u & 3) + 2 * (u >> 2));
    // [tile][chunk][lane][step]: a lane's four words of a chunk are one 16-byte load
    w5[(((int64_t)t * (s_pad >> 2) + (s >> 2)) * 64 + L) * 4 + (s & 3)] = o;
}

// int5 records as the int4 zero-point ones, the zero byte holding 16 - z as
// a signed byte (z - 1 = qzeros[s, n], a byte per group and column); rows
// past N and steps past K: scale 0, byte 0
__global__ __launch_bounds__(256) void prep_i5s_kernel(const uint16_t* __restrict__ sc, const uint8_t* __restrict__ qz,
                                                       int N, int K, int tiles, int c_pad, uint8_t* __restrict__ st) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)tiles * c_pad * 64) return;
    const int r = (int)(i & 15);
    const int u = (int)((i >> 4) & 3);
    const int64_t tc = i >> 6;
    const int c = (int)(tc % c_pad), t = (int)(tc / c_pad);
    const int s = 4 * c + u, n = 16 * t + r;
    const bool in = n < N && s < K / 128;
    uint8_t* rec = st + 256 * tc;
    const int e = 16 * (r >> 2) + 4 * u + (r & 3);
    reinterpret_cast<uint16_t*>(rec)[e] = in ? sc[(int64_t)s * N + n] : (uint16_t)0;
    rec[128 + e] = in ? (uint8_t)(int8_t)(15 - (int)qz[(int64_t)s * N + n]) : (uint8_t)0;
    rec[192 + e] = 0;
}

// ---------------------------------------------------------------------------
// decode band on prepared weights (M <= 32)
//
// Workgroup = TW x KW waves: TW 16-row weight tiles, each tile's K range cut into
// KW parts, one wave per (tile, part) -- many short contiguous weight streams
// (per wave a few KiB in 1 KiB load instructions) keep HBM busier than one long
// stream per tile.  The workgroup first copies the activations of its K range
// (all M rows) into LDS (rows padded by 16 bytes, so the 16 column lanes of an
// MFMA fragment hit distinct banks), then each wave streams its weight blocks
// and scale dwords through a D-deep register ring, loads issued D-1 chunks
// ahead of the MFMAs (straight-line code between scheduling barriers; chunk
// indices past the end re-read the last chunk rather than branching).  The KW
// partial accumulators of a tile are added through LDS in part order 0..KW-1
// (deterministic) by the part-0 wave, which writes the bf16 output -- or, when
// the grid also splits K across workgroups (ks > 1, for activations too large
// for LDS), fp32 partials that the group's last split to arrive adds in place.
// ---------------------------------------------------------------------------

struct PDecArgs {
    const uint8_t* x8;      // fp8 [M, K] (W4A4: e2m1 codes [M, K/2])
    const float* xs;        // token scales (W4A4: none)
    const uint8_t* xe;      // W4A4: activation e8m0 [M, K/32]
    const uint32_t* w5;     // int5: fifth-bit plane [tile][chunk][lane][step] words
    const uint16_t* xb;     // fused quant: bf16 activations, row stride ldx elements
    int64_t ldx;
    uint8_t* x8_out;        // fused quant: e4m3 codes [M, K] and token scales [M] written
    float* xs_out;          // by workgroup 0
    const uint4* wt;
    const uint8_t* st;      // e8m0 dwords (MXFP4) or fp16 row scales (int4), fragment order
    uint16_t* out;
    float* partials;
    uint32_t* counters;     // ks > 1: one arrival counter per group
    int sk_inplace;         // ks > 1: the last split reduces (else the reduction kernel does)
    int M, N, K;
    int s_pad, c_pad;   // padded 128-steps and 4-step chunks per row tile
    int tiles;          // 16-row tiles (ceil(N / 16))
    int tw, kw;         // tiles and K parts per workgroup
    int groups;         // workgroups per split (ceil(tiles / tw))
    int ks, c_per;      // K splits across workgroups, chunks per split
};

template <int WF> struct PChunk;
template <> struct PChunk<kWMx> {
    uint4 w[4];
    uint32_t s;          // e8m0 dword of the chunk
};
template <> struct PChunk<kWI4> {
    uint4 w[4];
    uint2 s[4];          // fp16 row scales of each step
};
template <> struct PChunk<kWMxA4> : PChunk<kWMx> {};
template <> struct PChunk<kWI4Z> {
    uint4 w[4];
    uint2 s[4];          // fp16 row scales of each step (the lane's four output rows)
    uint32_t z[4];       // bytes 16 - z of the same rows
};
template <> struct PChunk<kWI5> : PChunk<kWI4Z> {
    uint32_t b[4];       // fifth bits of each step's 32 codes
};

// chunk j of this wave's range: 4 weight blocks (sp: MXFP4 dwords of the
// tile's chunks, lane-indexed; int4 8-byte row-scale quads, (chunk, step, g))
template <int WF>
__device__ __forceinline__ void pdec_load(const uint4* wp, const void* sp, const uint32_t* bp, int j,
                                          PChunk<WF>& c) {
#pragma unroll
    for (int u = 0; u < 4; ++u) c.w[u] = load_stream16(wp + (4 * j + u) * 64);
    if constexpr (WF == kWI5) {
        // the lane's four plane words of chunk j
        const uint4 b = load_stream16(reinterpret_cast<const uint4*>(bp) + 64 * j);
        c.b[0] = b.x;
        c.b[1] = b.y;
        c.b[2] = b.z;
        c.b[3] = b.w;
    }
    if constexpr (WF == kWI4 || WF == kWI4Z || WF == kWI5) {
        // sp: the lane group's 32 scale bytes in the wave's first chunk
        // record (128 bytes per chunk, or 256 with the zero bytes 128 on)
        constexpr int kRec = WF == kWI4 ? 128 : 256;
        const uint8_t* rec = reinterpret_cast<const uint8_t*>(sp) + kRec * j;
        const uint4 s01 = *reinterpret_cast<const uint4*>(rec);
        const uint4 s23 = *reinterpret_cast<const uint4*>(rec + 16);
        c.s[0] = make_uint2(s01.x, s01.y);
        c.s[1] = make_uint2(s01.z, s01.w);
        c.s[2] = make_uint2(s23.x, s23.y);
        c.s[3] = make_uint2(s23.z, s23.w);
        if constexpr (WF != kWI4) {
            // the zero bytes: 16 per lane group, 128 + 16 q from the record
            const uint4 z = *reinterpret_cast<const uint4*>(rec + 128 - 16 * ((threadIdx.x & 63) >> 4));
            c.z[0] = z.x;
            c.z[1] = z.y;
            c.z[2] = z.z;
            c.z[3] = z.w;
        }
    } else {
        c.s = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(sp) + j * 64);
    }
}

// chunk j's products: activation rows from LDS (xl, stride; W4A4 codes 256 B
// per chunk, their e8m0 at xel, 16 B per chunk and row)
template <int MT, int WF>
__device__ __forceinline__ void pdec_compute(const uint8_t* xl, int stride, const uint8_t* xel, int estride,
                                             int lane, int M, int j, const PChunk<WF>& c, v4f (&acc)[MT]) {
    const int g = lane >> 4;
    if constexpr (WF == kWMxA4) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = min(mt * 16 + (lane & 15), M - 1);
            const uint4 e = *reinterpret_cast<const uint4*>(xel + m * estride + 16 * j);
            const uint8_t* p = xl + m * stride + 256 * j + 16 * g;
            const v8i b0 = frag_fp4(*reinterpret_cast<const uint4*>(p));
            const v8i b1 = frag_fp4(*reinterpret_cast<const uint4*>(p + 64));
            const v8i b2 = frag_fp4(*reinterpret_cast<const uint4*>(p + 128));
            const v8i b3 = frag_fp4(*reinterpret_cast<const uint4*>(p + 192));
            acc[mt] = mfma44<0>(frag_fp4(c.w[0]), b0, acc[mt], (int)c.s, (int)(e.x >> (8 * g)));
            acc[mt] = mfma44<1>(frag_fp4(c.w[1]), b1, acc[mt], (int)c.s, (int)(e.y >> (8 * g)));
            acc[mt] = mfma44<2>(frag_fp4(c.w[2]), b2, acc[mt], (int)c.s, (int)(e.z >> (8 * g)));
            acc[mt] = mfma44<3>(frag_fp4(c.w[3]), b3, acc[mt], (int)c.s, (int)(e.w >> (8 * g)));
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if constexpr (WF == kWMx) {
            const v8i aw = frag_fp4(c.w[u]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = min(mt * 16 + (lane & 15), M - 1);
                const uint8_t* p = xl + m * stride + 128 * (4 * j + u) + 16 * g;
                const v8i bx = frag_fp8(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 64));
                if (u == 0) acc[mt] = mfma16<0>(aw, bx, acc[mt], (int)c.s);
                if (u == 1) acc[mt] = mfma16<1>(aw, bx, acc[mt], (int)c.s);
                if (u == 2) acc[mt] = mfma16<2>(aw, bx, acc[mt], (int)c.s);
                if (u == 3) acc[mt] = mfma16<3>(aw, bx, acc[mt], (int)c.s);
            }
        } else if constexpr (kIsI4<WF> || WF == kWI5) {
            const I4Split w = i4_split(c.w[u]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = min(mt * 16 + (lane & 15), M - 1);
                const uint8_t* p = xl + m * stride + 128 * (4 * j + u) + 16 * g;
                const v8i bx = frag_fp8(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 64));
                if constexpr (WF == kWI5)
                    acc[mt] = i5_split_mma(w, i5_bit_frag(c.b[u]), bx, acc[mt], c.s[u], c.z[u]);
                else if constexpr (WF == kWI4Z)
                    acc[mt] = i4z_split_mma(w, bx, acc[mt], c.s[u], c.z[u]);
                else
                    acc[mt] = i4_split_mma(w, bx, acc[mt], c.s[u]);
            }
        }
    }
}

// activation elements q0 + u * nthreads (u < AB) of the workgroup's [M, kr]
// slice, 16 bytes each (16 fp8 values, or 32 e2m1 codes for W4A4)
template <bool A4, int AB>
__device__ __forceinline__ void pdec_act_load(const PDecArgs& a, int kbase, int per_row, int total, int q0,
                                              int nthreads, uint4 (&v)[AB]) {
    constexpr int kPer = A4 ? 32 : 16;
    const int64_t row_bytes = A4 ? a.K / 2 : a.K;
#pragma unroll
    for (int u = 0; u < AB; ++u) {
        const int q = q0 + u * nthreads;
        const int m = q / per_row, col = q - m * per_row;
        const int k = kbase + kPer * col;
        v[u] = (q < total && k < a.K)
                   ? *reinterpret_cast<const uint4*>(a.x8 + (int64_t)m * row_bytes + (A4 ? k / 2 : k))
                   : make_uint4(0, 0, 0, 0);
    }
}
// W4A4: the e8m0 of the workgroup's chunks -> LDS, 16 bytes per chunk and
// row (dword u = step u's four 32-wide blocks); blocks past K read as zero.
// Rows of e8m0 are K/32 bytes, a multiple of 4 but not always of 16: dword loads.
// Fused quant: the bf16 activations of the workgroup's (whole) K range,
// items of 8 values (16 bytes), q0 + u * nthreads for u < AB; items past K
// read as zero
// (every load issued, from an in-range address, and the out-of-range items
// zeroed afterwards: loads under branches leave the compiler's wait counts
// conservative, and the first use would then wait for the weight loads
// issued behind them)
template <int AB>
__device__ __forceinline__ void pdec_bf16_load(const PDecArgs& a, int per_row, int total, int q0, int nthreads,
                                               uint4 (&v)[AB]) {
#pragma unroll
    for (int u = 0; u < AB; ++u) {
        const int q = q0 + u * nthreads;
        const int qc = min(q, total - 1);
        const int m = qc / per_row, k = 8 * (qc - m * per_row);
        const uint4 t = *reinterpret_cast<const uint4*>(a.xb + (int64_t)m * a.ldx + min(k, a.K - 8));
        const bool ok = q < total && k < a.K;
        v[u] = make_uint4(ok ? t.x : 0u, ok ? t.y : 0u, ok ? t.z : 0u, ok ? t.w : 0u);
    }
}

// Fused quant: per-token e4m3 quantization of the loaded items into the LDS
// activation rows, by the rule of the standalone quant kernel (s = amax / 448,
// 1 for a zero row; code = e4m3 of x / s, nearest even, saturating): the row
// amax as the largest fp32 bit pattern of the items' non-negative maxima
// (fmaxf drops NaN as the standalone kernel's reduction does), reduced across
// the wave -- a row is a multiple of 64 items and a wave's 64 items of one
// batch are consecutive, so they share a row and are all valid or all past
// the end -- then one LDS max atomic per wave and batch; then every value
// divided by its row's scale.  amax_u: M words of LDS.
template <int AB>
__device__ __forceinline__ void pdec_fused_quant(const PDecArgs& a, uint8_t* xl, int stride, int per_row, int total,
                                                 int nthreads, const uint4 (&v)[AB], uint32_t* amax_u) {
    if ((int)threadIdx.x < a.M) amax_u[threadIdx.x] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < AB; ++u) {
        const int q = threadIdx.x + u * nthreads;
        if (q - (int)(threadIdx.x & 63) >= total) continue;   // the wave's first item: uniform
        const uint32_t d[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mx = fmaxf(mx, fabsf(bf16_to_f32(d[i] & 0xFFFFu)));
            mx = fmaxf(mx, fabsf(bf16_to_f32(d[i] >> 16)));
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        if ((threadIdx.x & 63) == 0) atomicMax(&amax_u[q / per_row], __float_as_uint(mx));
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < AB; ++u) {
        const int q = threadIdx.x + u * nthreads;
        if (q >= total) continue;
        const int m = q / per_row, col = q - m * per_row;
        const float amax = __uint_as_float(amax_u[m]);
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        const uint32_t d[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = f32_to_e4m3_rne_sat(bf16_to_f32(d[i] & 0xFFFFu) / sc);
            const uint32_t hi = f32_to_e4m3_rne_sat(bf16_to_f32(d[i] >> 16) / sc);
            o[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
        }
        *reinterpret_cast<uint2*>(xl + m * stride + 8 * col) = make_uint2(o[0], o[1]);
    }
}

__device__ __forceinline__ void pdec_e8_load(const PDecArgs& a, int kbase, int nch, uint8_t* xel, int estride,
                                             int nthreads) {
    const int total = a.M * nch;
    for (int q = threadIdx.x; q < total; q += nthreads) {
        const int m = q / nch, c = q - m * nch;
        const int k0 = kbase + 512 * c;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(a.xe + (int64_t)m * (a.K / 32)) + k0 / 128;
        uint4 v;
        v.x = k0 < a.K ? src[0] : 0u;
        v.y = k0 + 128 < a.K ? src[1] : 0u;
        v.z = k0 + 256 < a.K ? src[2] : 0u;
        v.w = k0 + 384 < a.K ? src[3] : 0u;
        *reinterpret_cast<uint4*>(xel + m * estride + 16 * c) = v;
    }
}
template <int AB>
__device__ __forceinline__ void pdec_act_store(uint8_t* xl, int stride, int per_row, int total, int q0,
                                               int nthreads, const uint4 (&v)[AB]) {
#pragma unroll
    for (int u = 0; u < AB; ++u) {
        const int q = q0 + u * nthreads;
        const int m = q / per_row, col = q - m * per_row;
        if (q < total) *reinterpret_cast<uint4*>(xl + m * stride + 16 * col) = v[u];
    }
}

// a tile's outputs (ks = 1: bf16 of s_m x acc; K split: fp32 partials, written
// through to the device's coherence point)
template <int MT, bool A4, bool FQ>
__device__ __forceinline__ void pdec_store(const PDecArgs& a, int split, int n0, int lane, const v4f (&acc)[MT],
                                           const float (&sm_fq)[MT]) {
    const bool vec = (a.N & 3) == 0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + (lane & 15);
        if (m >= a.M) continue;
        if (a.ks == 1) {
            float sm;
            if constexpr (A4) sm = 1.f;
            else if constexpr (FQ) sm = sm_fq[mt];
            else sm = a.xs[m];
            uint16_t* o = a.out + (int64_t)m * a.N + n0;
            if (vec) {
                const uint32_t h0 = f32_to_bf16_rne(sm * acc[mt][0]) | (f32_to_bf16_rne(sm * acc[mt][1]) << 16);
                const uint32_t h1 = f32_to_bf16_rne(sm * acc[mt][2]) | (f32_to_bf16_rne(sm * acc[mt][3]) << 16);
                *reinterpret_cast<uint2*>(o) = make_uint2(h0, h1);
            } else {
                for (int r = 0; r < 4; ++r)
                    if (n0 + r < a.N) o[r] = (uint16_t)f32_to_bf16_rne(sm * acc[mt][r]);
            }
        } else if (vec) {
            sk_put4(sk_rsrc(a.partials), 4u * (uint32_t)(((int64_t)split * a.M + m) * a.N + n0), acc[mt][0],
                    acc[mt][1], acc[mt][2], acc[mt][3]);
        } else {
            float* p = a.partials + ((int64_t)split * a.M + m) * a.N + n0;
            for (int r = 0; r < 4; ++r)
                if (n0 + r < a.N) sk_put(p + r, acc[mt][r]);
        }
    }
}

template <int MT, int D, int WF, int AB, bool FQ>
__global__ __launch_bounds__(1024) void pdec_kernel(PDecArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t xl[];
    const int tg = blockIdx.x % a.groups, split = blockIdx.x / a.groups;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nthreads = a.tw * a.kw * 64;
    const int t = tg * a.tw + wave % a.tw;
    const int part = wave / a.tw;
    const int c0 = split * a.c_per;
    const int c1 = min(a.c_pad, c0 + a.c_per);
    const int nch_wg = c1 > c0 ? c1 - c0 : 0;
    constexpr bool A4 = WF == kWMxA4;
    // LDS: activation rows of this K range, 16 bytes apart mod 128 (W4A4:
    // the code rows, then the e8m0 rows)
    const int kbase = c0 * 512, kr = nch_wg * 512, stride = (A4 ? kr / 2 : kr) + 16;
    const int estride = kr / 32 + 16;
    uint8_t* xel = xl + a.M * stride;
    // this wave's chunks within the workgroup's range: an even share, the
    // first (nch_wg % kw) parts one chunk longer
    const int base_n = nch_wg / a.kw, extra = nch_wg % a.kw;
    const int j0 = part * base_n + min(part, extra);
    const int nch = base_n + (part < extra ? 1 : 0);
    const bool active = t < a.tiles && nch > 0;

    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
    // idle waves (past the last tile, or a part with no chunks) still run the
    // prologue loads: point them at a valid chunk of a valid tile
    const int tc = min(t, a.tiles - 1);
    const int jb = nch > 0 ? j0 : 0;
    const uint4* wp = a.wt + ((int64_t)tc * a.s_pad + 4 * (int64_t)(c0 + jb)) * 64 + lane;
    // int5: the same lane's fifth-bit words (one per step)
    const uint32_t* bp = WF == kWI5 ? a.w5 + (((int64_t)tc * (a.s_pad >> 2) + c0 + jb) * 64 + lane) * 4 : nullptr;
    const void* sp;
    if constexpr (WF == kWI4)
        sp = a.st + ((int64_t)tc * a.c_pad + c0 + jb) * 128 + 32 * (lane >> 4);
    else if constexpr (WF == kWI4Z || WF == kWI5)
        sp = a.st + ((int64_t)tc * a.c_pad + c0 + jb) * 256 + 32 * (lane >> 4);
    else
        sp = reinterpret_cast<const uint32_t*>(a.st) + ((int64_t)tc * a.c_pad + c0 + jb) * 64 + lane;
    const int last = nch > 0 ? nch - 1 : 0;

    // Activations of this workgroup's K range -> LDS (columns >= K read as
    // zero), 16 bytes per thread and load, in batches of AB loads per
    // thread so that their latencies overlap.  The first batch is issued
    // before the weight ring prologue: its LDS writes then wait only for these
    // (L2-resident) loads while the weight loads stay in flight.
    // (fused quant: the bf16 activations instead, all in one batch, and K
    // not split across workgroups)
    const int per_row = FQ ? kr / 8 : (A4 ? kr / 32 : kr / 16), act_total = a.M * per_row;
    uint4 av[AB];
    if constexpr (FQ)
        pdec_bf16_load<AB>(a, per_row, act_total, threadIdx.x, nthreads, av);
    else
        pdec_act_load<A4, AB>(a, kbase, per_row, act_total, threadIdx.x, nthreads, av);
    __builtin_amdgcn_sched_barrier(0);
    PChunk<WF> ring[D];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) pdec_load<WF>(wp, sp, bp, min(d, last), ring[d]);
    __builtin_amdgcn_sched_barrier(0);
    [[maybe_unused]] uint32_t* amax_u = reinterpret_cast<uint32_t*>(xl + a.M * stride);   // fused quant: row amax
    if constexpr (FQ) {
        pdec_fused_quant<AB>(a, xl, stride, per_row, act_total, nthreads, av, amax_u);
    } else {
        pdec_act_store(xl, stride, per_row, act_total, threadIdx.x, nthreads, av);
        for (int q0 = threadIdx.x + AB * nthreads; q0 < act_total; q0 += AB * nthreads) {
            pdec_act_load<A4, AB>(a, kbase, per_row, act_total, q0, nthreads, av);
            pdec_act_store(xl, stride, per_row, act_total, q0, nthreads, av);
        }
    }
    if constexpr (A4) pdec_e8_load(a, kbase, nch_wg, xel, estride, nthreads);
    __syncthreads();
    // fused quant: this lane's token scales (the reduction below reuses the
    // LDS), and the codes and scales written out once, by workgroup 0
    [[maybe_unused]] float sm_fq[MT];
    if constexpr (FQ) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float amax = __uint_as_float(amax_u[min(mt * 16 + (lane & 15), a.M - 1)]);
            sm_fq[mt] = amax > 0.0f ? amax / 448.0f : 1.0f;
        }
        if (blockIdx.x == 0) {
            const int row16 = a.K / 16;
            for (int q = threadIdx.x; q < a.M * row16; q += nthreads) {
                const int m = q / row16, c = q - m * row16;
                *reinterpret_cast<uint4*>(a.x8_out + (int64_t)m * a.K + 16 * c) =
                    *reinterpret_cast<const uint4*>(xl + m * stride + 16 * c);
            }
            if ((int)threadIdx.x < a.M) {
                const float amax = __uint_as_float(amax_u[threadIdx.x]);
                a.xs_out[threadIdx.x] = amax > 0.0f ? amax / 448.0f : 1.0f;
            }
        }
    }

    // this part's first activation column
    const uint8_t* xw = xl + (A4 ? 256 : 512) * j0;
    const uint8_t* xew = xel + 16 * j0;
    if (active) {
        for (int j = 0; j < nch; j += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                pdec_load<WF>(wp, sp, bp, min(j + d + D - 1, last), ring[(d + D - 1) % D]);
                __builtin_amdgcn_sched_barrier(0);
                if (j + d < nch) pdec_compute<MT, WF>(xw, stride, xew, estride, lane, a.M, j + d, ring[d], acc);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // add the K parts of each tile through LDS, in part order (the part-0
    // wave of a tile writes it)
    bool writer = true;
    if (a.kw > 1) {
        __syncthreads();   // all waves are done reading activations
        float4* red = reinterpret_cast<float4*>(xl);   // [kw][tw][MT][64 lanes]
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            red[((part * a.tw + wave % a.tw) * MT + mt) * 64 + lane] =
                make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
        __syncthreads();
        writer = part == 0;
        if (writer) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                float4 tsum = red[((0 * a.tw + wave) * MT + mt) * 64 + lane];
                for (int q = 1; q < a.kw; ++q) {
                    const float4 v = red[((q * a.tw + wave) * MT + mt) * 64 + lane];
                    tsum.x = tsum.x + v.x;
                    tsum.y = tsum.y + v.y;
                    tsum.z = tsum.z + v.z;
                    tsum.w = tsum.w + v.w;
                }
                acc[mt] = v4f{tsum.x, tsum.y, tsum.z, tsum.w};
            }
        }
    }
    const int g = lane >> 4;
    const int n0 = 16 * t + 4 * g;
    if (writer && t < a.tiles && n0 < a.N) pdec_store<MT, A4, FQ>(a, split, n0, lane, acc, sm_fq);
    if (a.ks > 1 && a.sk_inplace) {
        // K split across workgroups: the group's last split to arrive adds the
        // partials of its columns (the flag word in the activation LDS, which
        // every wave is done with once the arrival's first barrier passes; a
        // static LDS word would not fit beside the full 160 KB dynamic range)
        if (sk_arrive(a.counters + tg, a.ks, reinterpret_cast<uint32_t*>(xl)))
            sk_reduce(a.partials, A4 ? nullptr : a.xs, a.M, a.N, a.ks, 16 * tg * a.tw,
                      min(a.N, 16 * (tg + 1) * a.tw), a.out, threadIdx.x, nthreads);
    }
}

template <int MT, int D, int WF, int AB, bool FQ = false>
hipError_t launch_pdec(const PDecArgs& a, size_t lds, hipStream_t stream) {
    static bool attr_set = false;   // raise the dynamic LDS cap once per process
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)pdec_kernel<MT, D, WF, AB, FQ>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((pdec_kernel<MT, D, WF, AB, FQ>), dim3(a.groups * a.ks), dim3(64 * a.tw * a.kw), lds,
                       stream, a);
    return hipGetLastError();
}

// the plan's kernel instance: activation tiles p.mt, ring depth p.u (2..4),
// activation loads per thread and batch p.ab (4 or 8)
template <int WF>
hipError_t launch_pdec_plan(const GemmPlan& p, const PDecArgs& a, size_t lds, hipStream_t stream) {
#define W4A8_PDEC(MT, D, AB) \
    if (p.mt == MT && p.u == D && p.ab == AB) return launch_pdec<MT, D, WF, AB>(a, lds, stream);
    W4A8_PDEC(1, 2, 4) W4A8_PDEC(1, 2, 8) W4A8_PDEC(1, 3, 4) W4A8_PDEC(1, 3, 8) W4A8_PDEC(1, 4, 4)
    W4A8_PDEC(1, 4, 8) W4A8_PDEC(2, 2, 4) W4A8_PDEC(2, 2, 8) W4A8_PDEC(2, 3, 4) W4A8_PDEC(2, 3, 8)
    W4A8_PDEC(2, 4, 4) W4A8_PDEC(2, 4, 8)
#undef W4A8_PDEC
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Register-streamed tiles (decode band beyond one 16-row activation tile).
//
// A workgroup of four waves covers 4 R 16-row weight tiles against every
// activation row (16 MT of them); each wave owns R tiles, so each weight
// fragment has exactly one consumer and goes from HBM straight into that
// wave's registers -- a ring of D two-step units, loaded D - 1 units ahead --
// never through LDS, whose capacity then holds no weight bytes in flight.  The
// activations, which all four waves read, go through a 3-stage LDS ring of two
// K steps (256 bytes per row, rows padded by 16 bytes so that the 16 column
// lanes of a fragment hit distinct banks): a unit's activation loads are
// issued three units ahead, before that unit's weight loads, stored to LDS two
// units ahead of their use, and published by one barrier per unit.  Vector
// memory loads complete in issue order, so the wait that an activation store
// needs never holds back the weight loads issued after it.  With few tiles
// the grid also splits K; the group's last split to arrive adds the fp32
// partials in place.
// ---------------------------------------------------------------------------

struct DtArgs {
    const uint8_t* x8;
    const float* xs;
    const uint4* wt;
    const uint32_t* st;
    uint16_t* out;
    float* partials;
    uint32_t* counters;   // ks > 1: one arrival counter per group
    int sk_inplace;       // ks > 1: the last split reduces (else the reduction kernel does)
    int M, N, K;
    int s_pad, c_pad, tiles;
    int groups;      // workgroups per K split
    int ks, h_per;   // K splits across workgroups; two-step units per split (even)
};
constexpr int kDtRow = 256 + 16;     // LDS bytes per activation row and stage
template <int MT> constexpr int kDtStage = 16 * MT * kDtRow;

__device__ __forceinline__ void dt_barrier() {
    // the stage's LDS stores done, then the workgroup barrier; the empty asm
    // keeps the compiler from moving LDS accesses across it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// unit h's activations (absolute two-step unit h): 16 MT rows x 16 items of
// 16 bytes, MT per thread (item i of a thread: threadIdx.x + 256 i); rows past
// M repeat row M - 1, columns past K (a padded last step, whose weight codes
// are zero) read the row's last 16 bytes.  Items are named members of a
// native vector type (a struct copy of uint4 would go through private memory),
// so that they stay in registers across the unit loop.
typedef uint32_t dt_u32x4 __attribute__((ext_vector_type(4)));
template <int MT>
struct DtAct {
    dt_u32x4 v0, v1, v2, v3;
};
template <int MT, int I>
__device__ __forceinline__ dt_u32x4& dt_item(DtAct<MT>& x) {
    if constexpr (I == 0) return x.v0;
    else if constexpr (I == 1) return x.v1;
    else if constexpr (I == 2) return x.v2;
    else return x.v3;
}
// items of a thread: it = threadIdx.x + 64 W I < 256 MT (MT x 16 rows x 16)
template <int MT, int W> constexpr int kDtItems = (4 * MT + W - 1) / W;
template <int MT, int W, int I>
__device__ __forceinline__ void dt_act_load_item(const DtArgs& a, int h, DtAct<MT>& x) {
    if constexpr (I < kDtItems<MT, W>) {
        const int it = threadIdx.x + 64 * W * I, r = min(it >> 4, 16 * MT - 1), q = it & 15;
        const int m = min(r, a.M - 1);
        const int k = min(256 * h + 16 * q, a.K - 16);
        dt_item<MT, I>(x) = *reinterpret_cast<const dt_u32x4*>(a.x8 + (int64_t)m * a.K + k);
    }
}
template <int MT, int W, int I>
__device__ __forceinline__ void dt_act_store_item(uint8_t* sb, DtAct<MT>& x) {
    if constexpr (I < kDtItems<MT, W>) {
        const int it = threadIdx.x + 64 * W * I, r = it >> 4, q = it & 15;
        // fewer items than threads (16 waves, one activation tile): the rest store nothing
        if (64 * W * kDtItems<MT, W> == 256 * MT || it < 256 * MT)
            *reinterpret_cast<dt_u32x4*>(sb + r * kDtRow + 16 * q) = dt_item<MT, I>(x);
    }
}
template <int MT, int W>
__device__ __forceinline__ void dt_act_load(const DtArgs& a, int h, DtAct<MT>& x) {
    dt_act_load_item<MT, W, 0>(a, h, x);
    dt_act_load_item<MT, W, 1>(a, h, x);
    dt_act_load_item<MT, W, 2>(a, h, x);
    dt_act_load_item<MT, W, 3>(a, h, x);
}
template <int MT, int W>
__device__ __forceinline__ void dt_act_store(uint8_t* sb, DtAct<MT>& x) {
    dt_act_store_item<MT, W, 0>(sb, x);
    dt_act_store_item<MT, W, 1>(sb, x);
    dt_act_store_item<MT, W, 2>(sb, x);
    dt_act_store_item<MT, W, 3>(sb, x);
}

template <int MT, int R, int U0>
__device__ __forceinline__ void dt_products(const uint8_t* sb, int lane, const uint4 (&w)[R][2], const uint32_t (&s)[R],
                                            v4f (&acc)[R][MT]) {
    const int g = lane >> 4;
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
        v8i bx[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint8_t* p = sb + (16 * mt + (lane & 15)) * kDtRow + 128 * uu + 16 * g;
            bx[mt] = frag_fp8(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 64));
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const v8i af = frag_fp4(w[r][uu]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (uu == 0) acc[r][mt] = mfma16<U0>(af, bx[mt], acc[r][mt], (int)s[r]);
                else acc[r][mt] = mfma16<U0 + 1>(af, bx[mt], acc[r][mt], (int)s[r]);
            }
        }
    }
}

// a wave's weights of one two-step unit: steps 2 h, 2 h + 1 of its R tiles
// (h relative to the split) and their chunk's e8m0 dwords
template <int R>
struct DtW {
    uint4 w[R][2];
    uint32_t s[R];
};
template <int R>
__device__ __forceinline__ void dt_wload(const uint4* const (&wp)[R], const uint32_t* const (&sp)[R], int h, DtW<R>& u) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
        u.w[r][0] = load_stream16(wp[r] + (2 * h) * 64);
        u.w[r][1] = load_stream16(wp[r] + (2 * h + 1) * 64);
        u.s[r] = __builtin_nontemporal_load(sp[r] + (h >> 1) * 64);
    }
}

// Unit y (ring slot d = y % 4): the loads of unit y + 3 (activations first,
// into the set of y + 1's parity), the store of unit y + 2's activations
// (loaded in unit y - 1, in the set of y's parity), the products of unit y, the
// barrier.  nh is uniform over the workgroup, so every wave takes the same
// branches and barriers.
template <int MT, int R, int W, int d>
__device__ __forceinline__ void dt_unit(const DtArgs& a, uint8_t* lds, int lane, int h0, int nh, int y,
                                        const uint4* const (&wp)[R], const uint32_t* const (&sp)[R],
                                        DtW<R> (&ring)[4], DtAct<MT>& av_even, DtAct<MT>& av_odd,
                                        v4f (&acc)[R][MT]) {
    if (y >= nh) return;
    const int last = nh - 1;
    const int yl = min(y + 3, last);
    if constexpr ((d & 1) == 0) dt_act_load<MT, W>(a, h0 + yl, av_odd);
    else dt_act_load<MT, W>(a, h0 + yl, av_even);
    dt_wload<R>(wp, sp, yl, ring[(d + 3) & 3]);
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* sb2 = lds + ((y + 2) % 3) * kDtStage<MT>;
    if constexpr ((d & 1) == 0) dt_act_store<MT, W>(sb2, av_even);
    else dt_act_store<MT, W>(sb2, av_odd);
    dt_products<MT, R, 2 * (d & 1)>(lds + (y % 3) * kDtStage<MT>, lane, ring[d].w, ring[d].s, acc);
    __builtin_amdgcn_sched_barrier(0);
    dt_barrier();
}

template <int MT, int R, int W, int D>
__global__ __launch_bounds__(64 * W) void dtile_kernel(DtArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    static_assert(D == 4, "the unit bookkeeping assumes a 4-deep weight ring");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4;
    const int tg = blockIdx.x % a.groups, split = blockIdx.x / a.groups;
    const int t0 = (tg * W + wave) * R;
    const int h0 = split * a.h_per;                     // even
    const int nh = min(a.s_pad / 2 - h0, a.h_per);      // >= 1 (host)
    const int last = nh - 1;
    const uint4* wp[R];
    const uint32_t* sp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int tt = min(t0 + r, a.tiles - 1);         // waves past the last tile stream a valid one
        wp[r] = a.wt + ((int64_t)tt * a.s_pad + 2 * h0) * 64 + lane;
        sp[r] = a.st + ((int64_t)tt * a.c_pad + h0 / 2) * 64 + lane;
    }
    v4f acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[r][mt] = v4f{0.f, 0.f, 0.f, 0.f};
    DtW<R> ring[D];
    DtAct<MT> av_even, av_odd;
    // prologue: units 0 and 1 staged, unit 2's activations and units 0..2's
    // weights in flight
    dt_act_load<MT, W>(a, h0, av_even);
    dt_act_load<MT, W>(a, h0 + min(1, last), av_odd);
#pragma unroll
    for (int d = 0; d < D - 1; ++d) dt_wload<R>(wp, sp, min(d, last), ring[d]);
    dt_act_store<MT, W>(lds, av_even);
    dt_act_store<MT, W>(lds + kDtStage<MT>, av_odd);
    dt_act_load<MT, W>(a, h0 + min(2, last), av_even);
    dt_barrier();
    for (int h = 0; h < nh; h += 4) {
        dt_unit<MT, R, W, 0>(a, lds, lane, h0, nh, h, wp, sp, ring, av_even, av_odd, acc);
        dt_unit<MT, R, W, 1>(a, lds, lane, h0, nh, h + 1, wp, sp, ring, av_even, av_odd, acc);
        dt_unit<MT, R, W, 2>(a, lds, lane, h0, nh, h + 2, wp, sp, ring, av_even, av_odd, acc);
        dt_unit<MT, R, W, 3>(a, lds, lane, h0, nh, h + 3, wp, sp, ring, av_even, av_odd, acc);
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int t = t0 + r;
        const int n0 = 16 * t + 4 * g;
        if (t >= a.tiles || n0 >= a.N) continue;
        const bool vec = (a.N & 3) == 0;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mt * 16 + (lane & 15);
            if (m >= a.M) continue;
            if (a.ks == 1) {
                const float sm = a.xs[m];
                uint16_t* o = a.out + (int64_t)m * a.N + n0;
                if (vec) {
                    const uint32_t h0w = f32_to_bf16_rne(sm * acc[r][mt][0]) | (f32_to_bf16_rne(sm * acc[r][mt][1]) << 16);
                    const uint32_t h1w = f32_to_bf16_rne(sm * acc[r][mt][2]) | (f32_to_bf16_rne(sm * acc[r][mt][3]) << 16);
                    *reinterpret_cast<uint2*>(o) = make_uint2(h0w, h1w);
                } else {
                    for (int q = 0; q < 4; ++q)
                        if (n0 + q < a.N) o[q] = (uint16_t)f32_to_bf16_rne(sm * acc[r][mt][q]);
                }
            } else if (vec) {
                sk_put4(sk_rsrc(a.partials), 4u * (uint32_t)(((int64_t)split * a.M + m) * a.N + n0), acc[r][mt][0],
                        acc[r][mt][1], acc[r][mt][2], acc[r][mt][3]);
            } else {
                float* pp = a.partials + ((int64_t)split * a.M + m) * a.N + n0;
                for (int q = 0; q < 4; ++q)
                    if (n0 + q < a.N) sk_put(pp + q, acc[r][mt][q]);
            }
        }
    }
    if (a.ks > 1 && a.sk_inplace) {
        // K split: the group's last split to arrive adds the partials of its columns
        __shared__ uint32_t last_flag;
        if (sk_arrive(a.counters + tg, a.ks, &last_flag)) {
            const int n_lo = 16 * tg * W * R, n_hi = min(a.N, 16 * (tg + 1) * W * R);
            sk_reduce(a.partials, a.xs, a.M, a.N, a.ks, n_lo, n_hi, a.out, threadIdx.x, 64 * W);
        }
    }
}

template <int MT, int R, int W>
hipError_t launch_dtile_inst(const DtArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((dtile_kernel<MT, R, W, 4>), dim3(a.groups * a.ks), dim3(64 * W), 3 * kDtStage<MT>,
                       stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Spread tiles (wide layers, decode band up to 64 rows): one workgroup of
// eight waves per CU and the layer's 16-row weight tiles dealt out evenly --
// a workgroup takes the floor or the ceiling of tiles / workgroups, a wave
// the floor or the ceiling of an eighth of that (gate_up, 2176 tiles on 256
// CUs: 8 or 9 per workgroup, 1 or 2 per wave) -- each over all of K, so
// there are no partial sums and no second pass.  (The tiled kernel's 256-row
// panels give the same layer 136 workgroups: 120 CUs idle.)
//
// Weights stream straight into a register ring D steps ahead: per tile and
// step one 16-byte load per lane (the 1 KiB fragment block, lane order =
// operand order) and the chunk's e8m0 dword.  The activation slice of a step
// (64 rows x 128 bytes; rows past M repeat row M - 1) goes global ->
// registers (one 16-byte item per thread, D + 1 steps ahead) -> a 4-stage
// LDS ring shared by the eight waves, rows 128 bytes with 16-byte chunk c of
// row r at c ^ ((r >> 1) & 7), so that a fragment read (16 rows x 4 chunk
// groups) hits every bank once.  One barrier per step.  Iteration s:
//   barrier (stores of step s + 1 visible; step s - 2's stage free)
//   LDS reads of step s + 1's fragments (into the other register set)
//   load of step s + D + 1's activation item; store of step s + 2's
//   products of step s (fragments read in iteration s - 1)
//   loads of step s + D's weights (into the ring slot step s just used)
// so the LDS latency hides under the matrix pipe, and two waves per SIMD
// overlap one's reads with the other's products.  Every load is an ordinary
// compiler-visible load; the activation item is issued ahead of the weights
// of the same iteration, so the wait before its store (two steps ahead of
// use) never drains weights newer than the next step's.
//
// The loop runs over the padded steps (the padding blocks hold zero codes,
// whose products are zero) in branch-free trips of D steps (the padded step
// count is a multiple of 4; D = 8 only where it is a multiple of 8);
// activation loads past K repeat the last real step.  A wave with fewer
// tiles than the most (R) runs its own copy of the loop with R - 1, chosen
// once per wave.
// ---------------------------------------------------------------------------
struct SpArgs {
    const uint8_t* x8;
    const float* xs;
    const uint4* wt;
    const uint32_t* st;
    uint16_t* out;
    int M, N, K;
    int s_pad, c_pad, tiles, steps;   // steps = K / 128 (real), s_pad = padded
    int groups;
    const uint16_t* xb;     // fused quant (one token): bf16 activations
    uint8_t* x8_out;        // fused quant: e4m3 codes [K] and token scale written
    float* xs_out;          // by workgroup 0
    int out16;              // output rows stored in 16-byte pieces through LDS (N % 8 == 0, out 16-byte aligned,
                            // the block M x 32 nt bytes within the stage ring)
    int64_t xrs, xss;       // activation codes: bytes between rows and between 128-wide steps
                            // (row-major K and 128; step-major 128 and 128 M)
    const uint8_t* xe;      // MXFP4 activations: e8m0 [M, K/32] (x8 then holds e2m1 codes [M, K/2])
    const uint32_t* w5;     // int5: the fifth-bit planes of the fragment-order weights
};
constexpr int kSpThreads = 512;
constexpr int kSpWaves = kSpThreads / 64;
constexpr int kSpStage = 64 * 128;
constexpr int kSpStages = 4;

// CS: the e8m0 dwords loaded once per 4-step chunk into two chunk slots (the
// next chunk's issued at the chunk start, before that step's weights),
// instead of with every step's weights
template <int R, int D>
struct SpRing {
    dt_u32x4 w[D][R];
    uint32_t s[D][R];
    uint32_t cs[2][R];
    dt_u32x4 cr[2][R];      // plain layout: the row's e8m0 dwords of the chunk's 4 steps
    dt_u32x4 w8[8][R];      // plain layout: weights as loaded, steps s .. s + 7
    dt_u32x4 wp[2][R];      // plain layout: weights of steps s, s + 1 in operand lane order
};

template <int MT>
__device__ __forceinline__ void sp_read(const uint8_t* stage, int lane, v8i (&F)[MT]) {
    const int g = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int r = 16 * mt + (lane & 15), sw = (r >> 1) & 7;
        const uint8_t* row = stage + 128 * r;
        F[mt] = frag_fp8(*reinterpret_cast<const uint4*>(row + 16 * (g ^ sw)),
                         *reinterpret_cast<const uint4*>(row + 16 * ((g + 4) ^ sw)));
    }
}

// this wave's per-lane sources and this thread's activation item
template <int R>
struct SpSrc {
    const uint4* wp[R];
    const uint32_t* sp[R];
    const uint8_t* xrow;     // activation row of this thread's item, at its chunk
    uint32_t xdst;           // the item's offset in a stage
    uint32_t sh;             // plain layout: bit offset of the lane's K block in an e8m0 dword (8 g)
    int perm;                // plain layout: byte address of the loading lane whose item this lane takes
    int x_last, w_last;      // last real step (activations), last padded step (weights)
    int64_t xss;             // bytes between the steps of an activation row
};

template <int R>
__device__ __forceinline__ dt_u32x4 sp_act(const SpSrc<R>& q, int j) {
    return *reinterpret_cast<const dt_u32x4*>(q.xrow + q.xss * min(j, q.x_last));
}

// PL: the plain layout ([N, K/2] codes, [N, K/32] e8m0), whose 16-byte lane
// items of a step lie 64 bytes apart along the row instead of in one 1 KiB block
template <int R, int D, bool CS, bool PL>
__device__ __forceinline__ void sp_wload(const SpSrc<R>& q, int j, SpRing<R, D>& ring, int slot) {
    j = min(j, q.w_last);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint4 v = load_stream16(q.wp[r] + (int64_t)j * 64);
        ring.w[slot][r] = dt_u32x4{v.x, v.y, v.z, v.w};
        if constexpr (!CS) ring.s[slot][r] = q.sp[r][(j >> 2) * 64];
    }
}
// chunk c's e8m0 dwords (clamped to the last chunk) into chunk slot `slot`;
// plain layout: the row's 16 bytes of steps 4c .. 4c + 3 (the lane's K block
// is byte g of each dword), taken apart where the products use them so that
// no wait follows the loads
template <int R, int D, bool PL>
__device__ __forceinline__ void sp_csload(const SpSrc<R>& q, int c, SpRing<R, D>& ring, int slot) {
    c = min(c, q.w_last >> 2);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if constexpr (PL) ring.cr[slot][r] = *reinterpret_cast<const dt_u32x4*>(q.sp[r] + 4 * c);
        else ring.cs[slot][r] = q.sp[r][c * 64];
    }
}

// plain layout: steps j0 .. j0 + 3 of every tile, issued together so that each
// row's 256 contiguous bytes are requested at once (one step's 64 bytes per
// row, sixteen rows 2.5 KB apart per load, read one at a time, made poor use
// of the DRAM pages); default cache policy, as a 128-byte line holds two steps
template <int R, int D>
__device__ __forceinline__ void sp_wload_pl(const SpSrc<R>& q, int j0, SpRing<R, D>& ring, int slot0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u)
            ring.w8[(slot0 + u) % 8][r] =
                *reinterpret_cast<const dt_u32x4*>(q.wp[r] + (int64_t)min(j0 + u, q.w_last) * 4);
}
// plain layout: the loading lane 4n + g holds row n's K block g (four lanes
// per 64 contiguous bytes); the operand wants it in lane n + 16g
template <int R, int D>
__device__ __forceinline__ void sp_permute(const SpSrc<R>& q, SpRing<R, D>& ring, int from, int to) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ring.wp[to][r][i] = (uint32_t)__builtin_amdgcn_ds_bpermute(q.perm, (int)ring.w8[from][r][i]);
}

// one step of the main loop; J = s mod the trip length (ring and activation
// slots, stage, fragment set and chunk slot are compile-time)
// fused quant (one token): step s's fragment from the resident quantized row
// (every column of the operand the same row: a broadcast read)
__device__ __forceinline__ void sp_read_row(const uint8_t* row, int lane, v8i (&F)[1]) {
    const int g = lane >> 4;
    F[0] = frag_fp8(*reinterpret_cast<const uint4*>(row + 16 * g), *reinterpret_cast<const uint4*>(row + 16 * (g + 4)));
}

template <int MT, int R, int D, bool CS, bool PL, bool FQ, int J>
__device__ __forceinline__ void sp_step(uint8_t* lds, int s, int lane, const SpSrc<R>& q, SpRing<R, D>& ring,
                                        dt_u32x4 (&av)[D], v8i (&F0)[MT], v8i (&F1)[MT], v4f (&acc)[R][MT]) {
    if constexpr (FQ) {
        // the row stays in LDS: no staging, no barrier
        const uint8_t* row = lds + 128 * min(s + 1, q.x_last);
        if constexpr ((J & 1) == 0) sp_read_row(row, lane, F1);
        else sp_read_row(row, lane, F0);
    } else {
        dt_barrier();
        if constexpr ((J & 1) == 0) sp_read<MT>(lds + ((J + 1) % kSpStages) * kSpStage, lane, F1);
        else sp_read<MT>(lds + ((J + 1) % kSpStages) * kSpStage, lane, F0);
        av[(J + 1) % D] = sp_act(q, s + D + 1);
        *reinterpret_cast<dt_u32x4*>(lds + ((J + 2) % kSpStages) * kSpStage + q.xdst) = av[(J + 2) % D];
    }
    // plain layout: step s + 1's weights into operand order, a step ahead of their products
    if constexpr (PL) sp_permute<R, D>(q, ring, (J + 1) % 8, (J + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const dt_u32x4 w = PL ? ring.wp[J & 1][r] : ring.w[J % D][r];
        const v8i af = frag_fp4(make_uint4(w[0], w[1], w[2], w[3]));
        // the scale operand's low byte (opsel 0) is this step's e8m0
        const int sc = PL ? (int)(ring.cr[(J / 4) % 2][r][J & 3] >> q.sh)
                          : (int)((CS ? ring.cs[(J / 4) % 2][r] : ring.s[J % D][r]) >> (8 * (J & 3)));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if constexpr ((J & 1) == 0) acc[r][mt] = mfma16<0>(af, F0[mt], acc[r][mt], sc);
            else acc[r][mt] = mfma16<0>(af, F1[mt], acc[r][mt], sc);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (PL) {
        // steps s + 4 .. s + 7 into the slots of steps s - 4 .. s - 1
        if constexpr (J % 4 == 0) sp_wload_pl<R, D>(q, s + 4, ring, (J + 4) % 8);
    } else {
        sp_wload<R, D, CS, PL>(q, s + D, ring, J % D);
    }
    if constexpr (CS && J % 4 == 0) sp_csload<R, D, PL>(q, s / 4 + 1, ring, (J / 4 + 1) % 2);
}

// the trip: D steps (per-step e8m0), or 8 with chunk slots (two chunks)
template <int D, bool CS> constexpr int kSpTrip = CS ? 8 : D;
template <int MT, int R, int D, bool CS, bool PL, bool FQ, int J>
__device__ __forceinline__ void sp_trip(uint8_t* lds, int s, int lane, const SpSrc<R>& q, SpRing<R, D>& ring,
                                        dt_u32x4 (&av)[D], v8i (&F0)[MT], v8i (&F1)[MT], v4f (&acc)[R][MT]) {
    if constexpr (J < kSpTrip<D, CS>) {
        sp_step<MT, R, D, CS, PL, FQ, J>(lds, s + J, lane, q, ring, av, F0, F1, acc);
        sp_trip<MT, R, D, CS, PL, FQ, J + 1>(lds, s, lane, q, ring, av, F0, F1, acc);
    }
}

// bf16 out = scale x sum for the wave's tiles w0 .. w0 + R - 1 (the
// workgroup's: t_lo .. t_lo + nt - 1); SM 0: the token's scale xs[m], 1: s
template <int MT, int R, int SM>
__device__ __forceinline__ void sp_epilogue(const SpArgs& a, uint8_t* lds, const v4f (&acc)[R][MT], int w0, int lane,
                                            int t_lo, int nt, float s) {
    const int g = lane >> 4;
    if (a.out16) {
        // the workgroup's output block (M rows x 16 nt columns of bf16) assembled
        // in LDS, then stored row by row in 16-byte pieces, consecutive lanes
        // along a row: whole 128-byte lines per store instead of sixteen 32-byte
        // pieces (the products' lane layout), which took the write-back of a
        // 64-row block 2-3 us longer at the end of the launch
        const int pitch = 32 * nt;
        __syncthreads();   // every wave past its last fragment read
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = mt * 16 + (lane & 15);
                if (m >= a.M) continue;
                const float sm = SM ? s : a.xs[m];
                const uint32_t h0 = f32_to_bf16_rne(sm * acc[r][mt][0]) | (f32_to_bf16_rne(sm * acc[r][mt][1]) << 16);
                const uint32_t h1 = f32_to_bf16_rne(sm * acc[r][mt][2]) | (f32_to_bf16_rne(sm * acc[r][mt][3]) << 16);
                *reinterpret_cast<uint2*>(lds + m * pitch + 32 * (w0 - t_lo + r) + 8 * g) = make_uint2(h0, h1);
            }
        }
        __syncthreads();
        // columns past N (the last tile's) are not stored; N is a multiple of 8
        const int cpr = (min(16 * nt, a.N - 16 * t_lo)) / 8;
        uint8_t* ob = reinterpret_cast<uint8_t*>(a.out + 16 * (int64_t)t_lo);
        for (int i = (int)threadIdx.x; i < a.M * cpr; i += kSpThreads) {
            const int row = i / cpr, ch = i - row * cpr;
            *reinterpret_cast<uint4*>(ob + 2 * (int64_t)row * a.N + 16 * ch) =
                *reinterpret_cast<const uint4*>(lds + row * pitch + 16 * ch);
        }
        return;
    }
    const bool vec = (a.N & 3) == 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int n0 = 16 * (w0 + r) + 4 * g;
        if (n0 >= a.N) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mt * 16 + (lane & 15);
            if (m >= a.M) continue;
            const float sm = SM ? s : a.xs[m];
            uint16_t* o = a.out + (int64_t)m * a.N + n0;
            if (vec) {
                const uint32_t h0 = f32_to_bf16_rne(sm * acc[r][mt][0]) | (f32_to_bf16_rne(sm * acc[r][mt][1]) << 16);
                const uint32_t h1 = f32_to_bf16_rne(sm * acc[r][mt][2]) | (f32_to_bf16_rne(sm * acc[r][mt][3]) << 16);
                *reinterpret_cast<uint2*>(o) = make_uint2(h0, h1);
            } else {
                for (int qq = 0; qq < 4; ++qq)
                    if (n0 + qq < a.N) o[qq] = (uint16_t)f32_to_bf16_rne(sm * acc[r][mt][qq]);
            }
        }
    }
}

// a wave's loop over its tiles w0 .. w0 + R - 1, then bf16 out = token scale x
// sum (the workgroup's tiles: t_lo .. t_lo + nt - 1)
template <int MT, int R, int D, bool CS, bool PL, bool FQ>
__device__ __forceinline__ void sp_run(const SpArgs& a, uint8_t* lds, int w0, int lane, int t_lo, int nt) {
    const int tid = threadIdx.x, g = lane >> 4;
    SpSrc<R> q;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if constexpr (PL) {
            // plain layout (rows past N clamped: they are not stored): lane 4n + g loads row 16 t + n's
            // K block g of a step; lane n + 16 g loads row 16 t + n's e8m0
            const int row = min(16 * (w0 + r) + (lane >> 2), a.N - 1);
            const int srow = min(16 * (w0 + r) + (lane & 15), a.N - 1);
            q.wp[r] = a.wt + (int64_t)row * (a.K / 32) + (lane & 3);
            q.sp[r] = a.st + (int64_t)srow * (a.K / 128);
        } else {
            q.wp[r] = a.wt + (int64_t)(w0 + r) * a.s_pad * 64 + lane;
            q.sp[r] = a.st + (int64_t)(w0 + r) * a.c_pad * 64 + lane;
        }
    }
    q.sh = 8u * g;
    q.perm = 4 * (4 * (lane & 15) + g);
    // this thread's activation item: row tid / 8 (clamped to M - 1), chunk tid % 8
    const int xr = tid >> 3, c = tid & 7;
    q.xrow = a.x8 + (int64_t)min(xr, a.M - 1) * a.xrs + 16 * c;
    q.xss = a.xss;
    q.xdst = 128u * xr + 16u * (c ^ ((xr >> 1) & 7));
    q.x_last = a.steps - 1;
    q.w_last = a.s_pad - 1;

    v4f acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[r][mt] = v4f{0.f, 0.f, 0.f, 0.f};
    SpRing<R, D> ring;
    dt_u32x4 av[D];
    v8i F0[MT], F1[MT];

    // prologue = iterations -D-1 .. -1 without products: activation items of
    // steps 0 .. D, weights of steps 0 .. D - 1, steps 0 and 1 stored, step
    // 0's fragments read
    if constexpr (CS) {
        // first, and pinned there: the loop's wait for a chunk slot also covers
        // the entry from here, and a load the scheduler sank to the end of the
        // prologue would make that wait drain every load in flight on every trip
        sp_csload<R, D, PL>(q, 0, ring, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    [[maybe_unused]] float sm_fq = 1.0f;
    if constexpr (FQ) {
        // fused quant, one token: its bf16 row (16-byte items tid and tid + 512
        // of K / 8 <= 1024) before the weight ring prologue, so that the
        // quantization waits only for these L2-resident loads
        const int items = a.K / 8;
        uint4 xv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int qi = tid + kSpThreads * u;
            const uint4 t = *reinterpret_cast<const uint4*>(a.xb + 8 * (int64_t)min(qi, items - 1));
            xv[u] = qi < items ? t : make_uint4(0u, 0u, 0u, 0u);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < D; ++k) sp_wload<R, D, CS, PL>(q, k, ring, k);
        __builtin_amdgcn_sched_barrier(0);
        // the standalone quant kernel's rule: s = amax / 448 (1 for a zero row),
        // code = e4m3 of x / s, nearest even, saturating; the amax as the
        // largest bit pattern of the non-negative maxima (fmaxf drops NaN)
        uint32_t* amax_u = reinterpret_cast<uint32_t*>(lds + a.K);
        if (tid == 0) *amax_u = 0u;
        __syncthreads();
        float mx = 0.0f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t d[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mx = fmaxf(mx, fabsf(bf16_to_f32(d[i] & 0xFFFFu)));
                mx = fmaxf(mx, fabsf(bf16_to_f32(d[i] >> 16)));
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        if (lane == 0) atomicMax(amax_u, __float_as_uint(mx));
        __syncthreads();
        const float amax = __uint_as_float(*amax_u);
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int qi = tid + kSpThreads * u;
            if (qi >= items) continue;
            const uint32_t d[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
            uint32_t o[2] = {0u, 0u};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = f32_to_e4m3_rne_sat(bf16_to_f32(d[i] & 0xFFFFu) / sc);
                const uint32_t hi = f32_to_e4m3_rne_sat(bf16_to_f32(d[i] >> 16) / sc);
                o[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
            }
            *reinterpret_cast<uint2*>(lds + 8 * qi) = make_uint2(o[0], o[1]);
            // the codes and the scale written out once, by workgroup 0
            if (blockIdx.x == 0) *reinterpret_cast<uint2*>(a.x8_out + 8 * (int64_t)qi) = make_uint2(o[0], o[1]);
        }
        if (blockIdx.x == 0 && tid == 0) a.xs_out[0] = sc;
        sm_fq = sc;
        __syncthreads();
        v8i f[1];
        sp_read_row(lds, lane, f);
        F0[0] = f[0];
    } else {
        av[0] = sp_act(q, 0);
#pragma unroll
        for (int k = 0; k < D; ++k) {
            av[(k + 1) % D] = sp_act(q, k + 1);
            if (k == D - 2) *reinterpret_cast<dt_u32x4*>(lds + q.xdst) = av[0];
            if constexpr (PL) {
                if (k == 0) sp_wload_pl<R, D>(q, 0, ring, 0);
            } else {
                sp_wload<R, D, CS, PL>(q, k, ring, k);
            }
        }
        dt_barrier();
        sp_read<MT>(lds, lane, F0);
        *reinterpret_cast<dt_u32x4*>(lds + kSpStage + q.xdst) = av[1];
        if constexpr (PL) sp_permute<R, D>(q, ring, 0, 0);
    }

    for (int s = 0; s < a.s_pad; s += kSpTrip<D, CS>)
        sp_trip<MT, R, D, CS, PL, FQ, 0>(lds, s, lane, q, ring, av, F0, F1, acc);

    sp_epilogue<MT, R, FQ ? 1 : 0>(a, lds, acc, w0, lane, t_lo, nt, sm_fq);
}

template <int MT, int R, int D, bool CS, bool PL, bool FQ>
__global__ __launch_bounds__(kSpThreads) void spread_kernel(SpArgs a) {
    static_assert(D == 4 || D == 8, "a trip is one turn of the ring and whole 4-step chunks");
    static_assert(!PL || CS, "plain layout: the e8m0 bytes are gathered once per chunk");
    static_assert(!FQ || (MT == 1 && !PL), "fused quant: one token, fragment order");
    static_assert(!CS || D == 4, "chunk slots one chunk ahead: the ring may be at most 4 steps deep (deeper, the "
                                 "wait for a chunk's dwords would drain weights of later steps)");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kSpStages * kSpStage];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);   // uniform: scalar branches
    // this workgroup's tiles, then this wave's (the host gives every wave 1 .. R)
    const int64_t T = a.tiles, G = a.groups;
    const int t_lo = (int)(T * blockIdx.x / G), n = (int)(T * (blockIdx.x + 1) / G) - t_lo;
    const int w0 = t_lo + wave * n / kSpWaves, nr = t_lo + (wave + 1) * n / kSpWaves - w0;
    if constexpr (R > 1) {
        if (nr < R) {
            sp_run<MT, R - 1, D, CS, PL, FQ>(a, lds, w0, lane, t_lo, n);
            return;
        }
    }
    sp_run<MT, R, D, CS, PL, FQ>(a, lds, w0, lane, t_lo, n);
}

template <int MT, int R, int D, bool CS, bool PL = false, bool FQ = false>
hipError_t launch_spread_inst(const SpArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((spread_kernel<MT, R, D, CS, PL, FQ>), dim3(a.groups), dim3(kSpThreads), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The spread tiles with MXFP4 activations (W4A4 on wide layers, M <= 64).
// The weight stream is the fp8 form's (register ring 4 steps deep, the tiles'
// e8m0 dwords once per 4-step chunk, trips of 8 steps), and so is the 4-stage
// LDS ring of activation steps with one barrier per step.  A stage holds a
// step's e2m1 codes, 64 B per row with the four 16-byte K blocks XOR-swizzled
// by (row >> 2) & 3 as in the fp4 tile kernel.  The rows' e8m0 sit in two
// chunk areas (even and odd 4-step chunks), [step % 4][row] dwords, so that a
// fragment's 16 rows read 16 consecutive dwords.
//
// Staging is coarser than the fp8 form's, because what limits these tiles at
// 64 rows is the number of distinct activation lines a CU requests per step:
// each of the 512 threads (row tid / 8, piece tid % 8) loads 16 code bytes
// every second step (the row's two steps are one 128-byte line: piece p is
// step p / 4's K block p % 4) and one e8m0 dword every fourth (the row's
// chunk is 16 bytes: piece p takes step p % 4's dword, pieces p and p + 4
// store copies), which is 48 lines per step instead of 128 with a step's 64
// code bytes and e8m0 dword loaded every step.  A pair of steps is loaded
// four steps ahead of its store (two pair slots), a chunk's dwords four steps
// ahead (two chunk slots); the products are fp4 x fp4 (16 cycles, half the
// fp8 one) with both scale operands: the weight's byte of the chunk dword and
// byte g (the lane's K block) of the row's activation dword.  No token scale:
// out = bf16(sum).
// ---------------------------------------------------------------------------
constexpr int kSa4Stage = 64 * 64;                 // a step's codes (64 rows)
constexpr int kSa4Area = 2 * 1024;                 // a chunk's e8m0: two copies of [4 steps][64 rows] dwords
constexpr int kSa4E = kSpStages * kSa4Stage;       // the two chunk areas follow the four stages

template <int R>
struct Sa4Src {
    SpSrc<R> w;              // the weight sources (wp, sp, w_last)
    const uint8_t* xrow;     // this thread's code bytes (its row, K block) of step 0
    const uint8_t* erow;     // its row's e8m0 (step 0's dword)
    uint32_t xdst, edst;     // its offsets from the first stage of a pair / in a chunk area
    int h, d;                // its step within a pair, within a chunk
    int x_last;              // last real step
};

// the thread's 16 code bytes of pair u (steps 2u, 2u + 1; clamped to the last
// real step); its dword of chunk c
template <int R>
__device__ __forceinline__ uint4 sa4_pair(const Sa4Src<R>& q, int u) {
    return *reinterpret_cast<const uint4*>(q.xrow + 64 * (int64_t)min(2 * u + q.h, q.x_last));
}
// the codes of the thread's step t as staged: zero past the last real step.
// The loop runs whole trips of 8 steps, which may pass the padded steps;
// there the weight loads repeat the last padded step, and the zero codes make
// those products zero.  (Selected at the store, where the loaded value is
// needed anyway: a select right after the load would wait for it there.)
template <int R>
__device__ __forceinline__ uint4 sa4_staged(const Sa4Src<R>& q, int t, uint4 v) {
    return t <= q.x_last ? v : make_uint4(0u, 0u, 0u, 0u);
}
template <int R>
__device__ __forceinline__ uint32_t sa4_chunk(const Sa4Src<R>& q, int c) {
    return *reinterpret_cast<const uint32_t*>(q.erow + 4 * (int64_t)min(4 * c + q.d, q.x_last));
}
// step t's fragments (stage t % 4) and activation scale operands (byte g of
// the row's dword in the low byte; chunk area (t / 4) % 2)
template <int MT>
__device__ __forceinline__ void sa4_read(const uint8_t* stage, const uint8_t* area, int t4, int lane, v8i (&F)[MT],
                                         int (&E)[MT]) {
    const int g = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int r = 16 * mt + (lane & 15);
        F[mt] = frag_fp4(*reinterpret_cast<const uint4*>(stage + 64 * r + 16 * (g ^ ((r >> 2) & 3))));
        E[mt] = (int)(*reinterpret_cast<const uint32_t*>(area + 256 * t4 + 4 * r) >> (8 * g));
    }
}

template <int MT, int R, int J>
__device__ __forceinline__ void sa4_step(uint8_t* lds, int s, int lane, const Sa4Src<R>& q, SpRing<R, 4>& ring,
                                         uint4 (&pv)[2], uint32_t (&ev)[2], v8i (&F0)[MT], v8i (&F1)[MT],
                                         int (&E0)[MT], int (&E1)[MT], v4f (&acc)[R][MT]) {
    dt_barrier();
    // step s + 1's operands
    {
        const uint8_t* stage = lds + ((J + 1) % kSpStages) * kSa4Stage;
        const uint8_t* area = lds + kSa4E + (((J + 1) / 4) % 2) * kSa4Area;
        if constexpr ((J & 1) == 0) sa4_read<MT>(stage, area, (J + 1) % 4, lane, F1, E1);
        else sa4_read<MT>(stage, area, (J + 1) % 4, lane, F0, E0);
    }
    if constexpr ((J & 1) == 0) {
        // steps s + 2, s + 3 into their stages (both last read before this
        // step's barrier), then the pair of steps s + 6, s + 7 into the slot
        constexpr int slot = (J / 2 + 1) % 2;
        *reinterpret_cast<uint4*>(lds + ((J + 2) % kSpStages) * kSa4Stage + q.xdst) =
            sa4_staged(q, s + 2 + q.h, pv[slot]);
        pv[slot] = sa4_pair(q, s / 2 + 3);
    }
    if constexpr (J % 4 == 2) {
        // the chunk of steps s + 2 .. s + 5 into its area (the chunk two
        // before it was last read at step s - 4), then the next chunk's dword
        // into the other slot (its previous chunk stored at step s - 4)
        constexpr int c = ((J + 2) / 4) % 2;
        *reinterpret_cast<uint32_t*>(lds + kSa4E + c * kSa4Area + q.edst) = ev[c];
        ev[1 - c] = sa4_chunk(q, (s + 2) / 4 + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const dt_u32x4 w = ring.w[J % 4][r];
        const v8i af = frag_fp4(make_uint4(w[0], w[1], w[2], w[3]));
        const int sc = (int)(ring.cs[(J / 4) % 2][r] >> (8 * (J & 3)));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if constexpr ((J & 1) == 0) acc[r][mt] = mfma44<0>(af, F0[mt], acc[r][mt], sc, E0[mt]);
            else acc[r][mt] = mfma44<0>(af, F1[mt], acc[r][mt], sc, E1[mt]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    sp_wload<R, 4, true, false>(q.w, s + 4, ring, J % 4);
    if constexpr (J % 4 == 0) sp_csload<R, 4, false>(q.w, s / 4 + 1, ring, (J / 4 + 1) % 2);
}
template <int MT, int R, int J>
__device__ __forceinline__ void sa4_trip(uint8_t* lds, int s, int lane, const Sa4Src<R>& q, SpRing<R, 4>& ring,
                                         uint4 (&pv)[2], uint32_t (&ev)[2], v8i (&F0)[MT], v8i (&F1)[MT],
                                         int (&E0)[MT], int (&E1)[MT], v4f (&acc)[R][MT]) {
    if constexpr (J < 8) {
        sa4_step<MT, R, J>(lds, s + J, lane, q, ring, pv, ev, F0, F1, E0, E1, acc);
        sa4_trip<MT, R, J + 1>(lds, s, lane, q, ring, pv, ev, F0, F1, E0, E1, acc);
    }
}

template <int MT, int R>
__device__ __forceinline__ void sa4_run(const SpArgs& a, uint8_t* lds, int w0, int lane, int t_lo, int nt) {
    const int tid = threadIdx.x;
    Sa4Src<R> q;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        q.w.wp[r] = a.wt + (int64_t)(w0 + r) * a.s_pad * 64 + lane;
        q.w.sp[r] = a.st + (int64_t)(w0 + r) * a.c_pad * 64 + lane;
    }
    q.w.w_last = a.s_pad - 1;
    // this thread's staging items: row tid / 8 (clamped to M - 1), piece tid % 8
    const int xr = tid >> 3, pc = tid & 7;
    const int64_t row = min(xr, a.M - 1);
    q.h = pc >> 2;
    q.d = pc & 3;
    q.xrow = a.x8 + row * (a.K / 2) + 16 * (pc & 3);
    q.erow = a.xe + row * (a.K / 32);
    q.xdst = (uint32_t)(q.h * kSa4Stage + 64 * xr + 16 * ((pc & 3) ^ ((xr >> 2) & 3)));
    q.edst = (uint32_t)(q.h * 1024 + 256 * q.d + 4 * xr);
    q.x_last = a.steps - 1;

    v4f acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[r][mt] = v4f{0.f, 0.f, 0.f, 0.f};
    SpRing<R, 4> ring;
    uint4 pv[2];
    uint32_t ev[2];
    v8i F0[MT], F1[MT];
    int E0[MT], E1[MT];

    // prologue: chunk 0's weight dwords first (as in the fp8 form), the
    // activations of steps 0 .. 5 and chunks 0 and 1, the weights of steps
    // 0 .. 3; steps 0, 1 and chunk 0 stored, step 0's operands read.  Then
    // the loop's invariant holds at s = 0: slots hold pairs (2, 3), (4, 5) and
    // chunk 1
    sp_csload<R, 4, false>(q.w, 0, ring, 0);
    __builtin_amdgcn_sched_barrier(0);
    const uint4 p01 = sa4_pair(q, 0);
    const uint32_t e0 = sa4_chunk(q, 0);
    pv[1] = sa4_pair(q, 1);
    ev[1] = sa4_chunk(q, 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) sp_wload<R, 4, true, false>(q.w, k, ring, k);
    *reinterpret_cast<uint4*>(lds + q.xdst) = sa4_staged(q, q.h, p01);
    *reinterpret_cast<uint32_t*>(lds + kSa4E + q.edst) = e0;
    pv[0] = sa4_pair(q, 2);
    dt_barrier();
    sa4_read<MT>(lds, lds + kSa4E, 0, lane, F0, E0);

    for (int s = 0; s < a.s_pad; s += 8) sa4_trip<MT, R, 0>(lds, s, lane, q, ring, pv, ev, F0, F1, E0, E1, acc);
    sp_epilogue<MT, R, 1>(a, lds, acc, w0, lane, t_lo, nt, 1.0f);
}

template <int MT, int R>
__global__ __launch_bounds__(kSpThreads) void spread_a4_kernel(SpArgs a) {
    static_assert(kSa4E + 2 * kSa4Area <= kSpStages * kSpStage, "the stages and chunk areas fit the ring's LDS");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kSpStages * kSpStage];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int64_t T = a.tiles, G = a.groups;
    const int t_lo = (int)(T * blockIdx.x / G), n = (int)(T * (blockIdx.x + 1) / G) - t_lo;
    const int w0 = t_lo + wave * n / kSpWaves, nr = t_lo + (wave + 1) * n / kSpWaves - w0;
    if constexpr (R > 1) {
        if (nr < R) {
            sa4_run<MT, R - 1>(a, lds, w0, lane, t_lo, n);
            return;
        }
    }
    sa4_run<MT, R>(a, lds, w0, lane, t_lo, n);
}

// ---------------------------------------------------------------------------
// The spread tiles with int4 g128 weights (wide layers, M <= 64; WF: kWI4,
// kWI4Z with a zero point per group and row, or kWI5, int5 codes).
// Weight blocks, activation staging and trips are the fp8 form's (register
// ring 4 steps deep, 4-stage LDS ring of e4m3 steps, trips of 8 steps).  The
// products are the split-K decode kernel's: each code taken as two e2m1
// fragments (c & 3 and (c >> 2) & 3, scaled by 2 and 8 through the e8m0
// operand) on top of the -8 sum(x) term from a constant fragment, which is
// taken once per activation tile and step for all of the wave's tiles; the
// step's fp16 row scales multiply the sum in fp32.  The row scales of a
// 4-step chunk (the lane's four output rows x four steps: 32 bytes of the
// tile's 128-byte record) are loaded once per chunk into two chunk slots, as
// the fp8 form's e8m0 dwords.  Where the chunk count is odd the last trip
// passes the padded steps by four; the staged activation codes are zero there
// (selected at the LDS store), so those products add nothing.  kWI4Z: the
// records are 256 bytes (the scales, then bytes 16 - z in the same order) and
// the products add (8 - z) sum(x) per row before its scale, sum(x) being
// -1/8 of the constant product.  kWI5: records as kWI4Z with signed bytes
// 16 - z; c - 16 = 2 (c & 3)/2 + 8 ((c >> 2) & 3)/2 + 16 b4 - 16 takes a
// third product on the fifth bits (the lane's four plane words of a chunk
// loaded with its scales), the constant product is -16 sum(x), and each row
// adds (16 - z) sum(x).
// ---------------------------------------------------------------------------
template <int R>
struct Si4Scales {
    const uint4* p[R];       // the lane's 32 bytes of scales in chunk 0's record, per tile
    const uint4* z[R];       // kWI4Z / kWI5: the lane's 16 zero bytes in chunk 0's record
    const uint4* b[R];       // kWI5: the lane's four fifth-bit plane words of chunk 0
    int c_last;              // last padded chunk
};
// chunk c's slot: the lane's scales (2 x 16 bytes), with zero points also its
// 16 zero bytes, int5 also its plane words
template <int R, int WF>
__device__ __forceinline__ void si4_csload(const Si4Scales<R>& q, int c, uint4 (&cs)[R][4]) {
    c = min(c, q.c_last);
    constexpr int rec = WF == kWI4 ? 8 : 16;   // record size in 16-byte units
#pragma unroll
    for (int r = 0; r < R; ++r) {
        cs[r][0] = q.p[r][rec * c];
        cs[r][1] = q.p[r][rec * c + 1];
        if constexpr (WF != kWI4) cs[r][2] = q.z[r][rec * c];
        if constexpr (WF == kWI5) cs[r][3] = q.b[r][64 * c];
    }
}
// The int5 tiles with four activation tiles and two weight tiles per wave hold
// too much for 256 registers with the chunk slots (64 of them); they take each
// step's side data with its weights instead, one ring slot per step: the two
// fp16 scale pairs, the zero-byte dword and the plane word (32 registers)
template <int MT, int R, int WF> constexpr bool kSi4Step = WF == kWI5 && MT == 4 && R == 2;
template <int R>
__device__ __forceinline__ void si4_sdload(const Si4Scales<R>& q, int j, int w_last, uint4 (&sd)[R]) {
    j = min(j, w_last);
    const int c = j >> 2, u = j & 3;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint2 sc = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(q.p[r]) + 256 * c + 8 * u);
        const uint32_t zb = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(q.z[r]) + 256 * c + 4 * u);
        const uint32_t pw = reinterpret_cast<const uint32_t*>(q.b[r] + 64 * (int64_t)c)[u];
        sd[r] = make_uint4(sc.x, sc.y, zb, pw);
    }
}
__device__ __forceinline__ void si4_stage(uint8_t* stage, const SpSrc<1>& q, int t, dt_u32x4 v) {
    *reinterpret_cast<dt_u32x4*>(stage + q.xdst) = t <= q.x_last ? v : dt_u32x4{0u, 0u, 0u, 0u};
}

template <int MT, int R, int WF, int J>
__device__ __forceinline__ void si4_step(uint8_t* lds, int s, int lane, const SpSrc<1>& xq, const SpSrc<R>& q,
                                         const Si4Scales<R>& sq, SpRing<R, 4>& ring, uint4 (&cs)[2][R][4],
                                         uint4 (&sd)[4][R], dt_u32x4 (&av)[4], v8i (&F0)[MT], v8i (&F1)[MT],
                                         v4f (&acc)[R][MT]) {
    constexpr bool PS = kSi4Step<MT, R, WF>;
    constexpr int kX2 = 128, kX8 = 130, kX16 = 131;   // e8m0 2^1, 2^3, 2^4
    constexpr int kXc = WF == kWI5 ? kX16 : kX8;      // the constant product: -16 or -8 sum(x)
    dt_barrier();
    if constexpr ((J & 1) == 0) sp_read<MT>(lds + ((J + 1) % kSpStages) * kSpStage, lane, F1);
    else sp_read<MT>(lds + ((J + 1) % kSpStages) * kSpStage, lane, F0);
    av[(J + 1) % 4] = sp_act(xq, s + 5);
    si4_stage(lds + ((J + 2) % kSpStages) * kSpStage, xq, s + 2, av[(J + 2) % 4]);
    __builtin_amdgcn_sched_barrier(0);
    const v8i neg1 = {(int)0xAAAAAAAA, (int)0xAAAAAAAA, (int)0xAAAAAAAA, (int)0xAAAAAAAA, 0, 0, 0, 0};
    v4f t0[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        t0[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(neg1, (J & 1) == 0 ? F0[mt] : F1[mt],
                                                                  v4f{0.f, 0.f, 0.f, 0.f}, kFmtFp4, kFmtFp8, 0, kXc,
                                                                  0, kUnitScale);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const dt_u32x4 wv = ring.w[J % 4][r];
        const I4Split w = i4_split(make_uint4(wv[0], wv[1], wv[2], wv[3]));
        const uint4 sv = PS ? sd[J % 4][r] : cs[(J / 4) % 2][r][(J & 3) / 2];
        const uint32_t s01 = PS || (J & 1) == 0 ? sv.x : sv.z, s23 = PS || (J & 1) == 0 ? sv.y : sv.w;
        const float s4[4] = {f16_to_f32(s01 & 0xFFFFu), f16_to_f32(s01 >> 16), f16_to_f32(s23 & 0xFFFFu),
                             f16_to_f32(s23 >> 16)};
        // zero points: the row's zero term over the constant product, (8 - z) / -8
        // (int4, bytes 16 - z) or (16 - z) / -16 (int5, signed bytes 16 - z)
        float zf[4] = {0.f, 0.f, 0.f, 0.f};
        v8i b4 = {0, 0, 0, 0, 0, 0, 0, 0};
        if constexpr (WF != kWI4) {
            const uint4 zv = cs[(J / 4) % 2][r][2];
            const uint32_t zb = PS ? sd[J % 4][r].z
                                   : (J & 3) == 0 ? zv.x : (J & 3) == 1 ? zv.y : (J & 3) == 2 ? zv.z : zv.w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (WF == kWI5) zf[i] = (float)(int)(int8_t)((zb >> (8 * i)) & 0xFFu) * -0.0625f;
                else zf[i] = (float)((int)((zb >> (8 * i)) & 0xFFu) - 8) * -0.125f;
            }
        }
        if constexpr (WF == kWI5) {
            const uint4 bv = cs[(J / 4) % 2][r][3];
            b4 = i5_bit_frag(PS ? sd[J % 4][r].w
                                : (J & 3) == 0 ? bv.x : (J & 3) == 1 ? bv.y : (J & 3) == 2 ? bv.z : bv.w);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const v8i bx = (J & 1) == 0 ? F0[mt] : F1[mt];
            v4f t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.lo, bx, t0[mt], kFmtFp4, kFmtFp8, 0, kX2, 0,
                                                                     kUnitScale);
            t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.hi, bx, t, kFmtFp4, kFmtFp8, 0, kX8, 0,
                                                                 kUnitScale);
            if constexpr (WF == kWI5)
                t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b4, bx, t, kFmtFp4, kFmtFp8, 0, kX16, 0,
                                                                     kUnitScale);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float u = WF != kWI4 ? __builtin_fmaf(zf[i], t0[mt][i], t[i]) : t[i];
                acc[r][mt][i] = __builtin_fmaf(s4[i], u, acc[r][mt][i]);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    sp_wload<R, 4, true, false>(q, s + 4, ring, J % 4);
    if constexpr (PS) si4_sdload<R>(sq, s + 4, q.w_last, sd[J % 4]);
    else if constexpr (J % 4 == 0) si4_csload<R, WF>(sq, s / 4 + 1, cs[(J / 4 + 1) % 2]);
}
template <int MT, int R, int WF, int J>
__device__ __forceinline__ void si4_trip(uint8_t* lds, int s, int lane, const SpSrc<1>& xq, const SpSrc<R>& q,
                                         const Si4Scales<R>& sq, SpRing<R, 4>& ring, uint4 (&cs)[2][R][4],
                                         uint4 (&sd)[4][R], dt_u32x4 (&av)[4], v8i (&F0)[MT], v8i (&F1)[MT],
                                         v4f (&acc)[R][MT]) {
    if constexpr (J < 8) {
        si4_step<MT, R, WF, J>(lds, s + J, lane, xq, q, sq, ring, cs, sd, av, F0, F1, acc);
        si4_trip<MT, R, WF, J + 1>(lds, s, lane, xq, q, sq, ring, cs, sd, av, F0, F1, acc);
    }
}

template <int MT, int R, int WF>
__device__ __forceinline__ void si4_run(const SpArgs& a, uint8_t* lds, int w0, int lane, int t_lo, int nt) {
    const int tid = threadIdx.x, g = lane >> 4;
    SpSrc<R> q;          // weights: blocks of tiles w0 .. w0 + R - 1
    Si4Scales<R> sq;     // their row-scale records
    const uint8_t* st = reinterpret_cast<const uint8_t*>(a.st);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        q.wp[r] = a.wt + (int64_t)(w0 + r) * a.s_pad * 64 + lane;
        const uint8_t* rec = st + (int64_t)(w0 + r) * a.c_pad * (WF == kWI4 ? 128 : 256);
        sq.p[r] = reinterpret_cast<const uint4*>(rec + 32 * g);
        sq.z[r] = reinterpret_cast<const uint4*>(rec + 128 + 16 * g);
        // int5 planes [tile][chunk][lane][step]: 16 bytes per lane and chunk
        sq.b[r] = WF == kWI5 ? reinterpret_cast<const uint4*>(a.w5) + (int64_t)(w0 + r) * a.c_pad * 64 + lane
                             : nullptr;
    }
    q.w_last = a.s_pad - 1;
    sq.c_last = a.c_pad - 1;
    // this thread's activation item: row tid / 8 (clamped to M - 1), chunk tid % 8
    SpSrc<1> xq;
    const int xr = tid >> 3, c = tid & 7;
    xq.xrow = a.x8 + (int64_t)min(xr, a.M - 1) * a.xrs + 16 * c;
    xq.xss = a.xss;
    xq.xdst = 128u * xr + 16u * (c ^ ((xr >> 1) & 7));
    xq.x_last = a.steps - 1;

    v4f acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[r][mt] = v4f{0.f, 0.f, 0.f, 0.f};
    SpRing<R, 4> ring;
    uint4 cs[2][R][4];   // chunk slots (unused with per-step side data)
    uint4 sd[4][R];      // per-step side data (kSi4Step only)
    dt_u32x4 av[4];
    v8i F0[MT], F1[MT];
    constexpr bool PS = kSi4Step<MT, R, WF>;

    // prologue as the fp8 form's: chunk 0's scales first, then the items of
    // steps 0 .. 4 and the weights of steps 0 .. 3; steps 0 and 1 staged, step
    // 0's fragments read
    if constexpr (!PS) si4_csload<R, WF>(sq, 0, cs[0]);
    __builtin_amdgcn_sched_barrier(0);
    av[0] = sp_act(xq, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        av[(k + 1) % 4] = sp_act(xq, k + 1);
        if (k == 2) si4_stage(lds, xq, 0, av[0]);
        sp_wload<R, 4, true, false>(q, k, ring, k);
        if constexpr (PS) si4_sdload<R>(sq, k, q.w_last, sd[k]);
    }
    dt_barrier();
    sp_read<MT>(lds, lane, F0);
    si4_stage(lds + kSpStage, xq, 1, av[1]);

    for (int s = 0; s < a.s_pad; s += 8)
        si4_trip<MT, R, WF, 0>(lds, s, lane, xq, q, sq, ring, cs, sd, av, F0, F1, acc);
    sp_epilogue<MT, R, 0>(a, lds, acc, w0, lane, t_lo, nt, 1.0f);
}

template <int MT, int R, int WF>
__global__ __launch_bounds__(kSpThreads) void spread_i4_kernel(SpArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kSpStages * kSpStage];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int64_t T = a.tiles, G = a.groups;
    const int t_lo = (int)(T * blockIdx.x / G), n = (int)(T * (blockIdx.x + 1) / G) - t_lo;
    const int w0 = t_lo + wave * n / kSpWaves, nr = t_lo + (wave + 1) * n / kSpWaves - w0;
    if constexpr (R > 1) {
        if (nr < R) {
            si4_run<MT, R - 1, WF>(a, lds, w0, lane, t_lo, n);
            return;
        }
    }
    si4_run<MT, R, WF>(a, lds, w0, lane, t_lo, n);
}

// fused-quant instances: one 16-row activation tile, the bf16 slice in one
// batch of 4 loads per thread (ring depth 2 or 3) or 8 (depth 2)
template <int WF>
hipError_t launch_pdec_fused(const GemmPlan& p, const PDecArgs& a, size_t lds, hipStream_t stream) {
    if (p.mt != 1 || p.ks != 1) return hipErrorInvalidValue;
    if (p.u == 2 && p.ab == 4) return launch_pdec<1, 2, WF, 4, true>(a, lds, stream);
    if (p.u == 2 && p.ab == 8) return launch_pdec<1, 2, WF, 8, true>(a, lds, stream);
    if (p.u == 3 && p.ab == 4) return launch_pdec<1, 3, WF, 4, true>(a, lds, stream);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// tiled band on prepared weights: BN (256 or 128) weight rows x BM (64, 128
// or 256) activation rows per workgroup, K in 128-wide steps through an
// NS-stage LDS ring (5 / 4 / 3 stages for BM = 64 / 128 / 256).
//
// Eight waves in an NWN x NWM grid; wave tile = 16*FN weight rows x 16*FM
// activation rows of 16x16x128 MFMAs.  Every stage is filled with direct
// global -> LDS copies (buffer loads with the LDS bit, 1 KiB per wave
// instruction, no registers): the BN/16 weight fragment blocks of the panel
// (lane order = MFMA order, read back with one conflict-free ds_read_b128 per
// fragment) and the BM x 128 activation slice, whose 16-byte chunk c of row r
// sits at chunk position c ^ ((r >> 1) & 7) (so the 16 rows of a fragment
// read land in 16 distinct bank groups).  The e8m0 dwords of a 4-step chunk
// (256 B per weight tile) go to one of two buffers of their own.  LDS offsets
// start at 256: a direct-to-LDS destination of address 0 would be taken for
// a null pointer by the address-space cast.
// ---------------------------------------------------------------------------

struct PfArgs {
    const uint8_t* x8;
    const float* xs;
    const uint8_t* wt;
    const uint8_t* st;
    uint16_t* out;
    int M, N, K;
    int ldo;                    // output row stride (N, or the whole layer's width for a column range)
    int s_pad, c_pad, tiles16;
    int tiles_m, tiles_n;
    int group_m;                // M tiles per group of the tile order
    int ks, s_per;              // K splits (steps s_per each, a multiple of 4; ks = 1: none)
    float* partials;            // ks > 1: fp32 [ks][M][N], token scale not applied
    const uint8_t* xe;          // W4A4: activation e8m0 [M, K/32] (x8 then holds e2m1 [M, K/2])
    const uint32_t* w5;         // int5: fifth-bit plane [tile][chunk][lane][step]
    const float* rs;            // int5: activation sums [chunk][M][4 steps] (fp32)
};

constexpr int kPfThreads = 512;
constexpr int kPfBase = 256;

// Direct global -> LDS copies through buffer loads with the LDS bit: lane L's
// 16 (4) bytes land at M0 + 16 L (4 L).  The buffer form moves L2-resident
// data into LDS at about twice the rate of the global form on gfx950
// (measured: ~32 vs ~14.5 TB/s aggregate for 1 KiB copies).  Issued through
// inline asm (M0 set in the same statement) so that the compiler's wait
// insertion does not treat them as LDS stores of unknown address -- it would
// otherwise drain every copy in flight before each LDS read.  Their
// completion is awaited explicitly (wait_vmcnt, then a barrier) before the
// stage they fill is read; loads complete in issue order, so the compiler's
// own vmcnt waits for other loads stay correct.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// raw buffer descriptor: 48-bit base, stride 0, `bytes` records (reads past
// them return zero), dword 3 = 32-bit data format as for every gfx9 buffer
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)n);
    r[3] = 0x00020000;
    return r;
}
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ void lds_dma16(const i32x4& rs, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 ::"v"(voff), "s"(rs), "s"(soff), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const i32x4& rs, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 ::"v"(voff), "s"(rs), "s"(soff), "s"(lds) : "memory", "m0");
}

// Stage sizes and the waves' share of the output tile.  MXFP4: NWM x NWN waves
// over (M, N), each with FN weight and FM activation fragments per step.
// int4: one wave row (NWM = 1), so that each wave widens only its FN = BN/128
// weight fragments per step and uses each against FM = BM/16 activation
// fragments (the widening and the per-step scaling are vector-ALU work that
// the MXFP4 format does inside the matrix instruction).
template <int BM, int BN, int WF = 0>
struct PfShape {
    static constexpr int NWM = kWiden<WF> ? 1 : (BM >= 256 ? 4 : (BM >= 128 ? 2 : 1));
    static constexpr int NWN = 8 / NWM;
    static constexpr int FN = BN / (16 * NWN);
    static constexpr int FM = BM / (16 * NWM);
    static constexpr int WBYTES = BN / 16 * 1024;      // weight blocks per stage
    static constexpr int ABYTES = BM * 128;                // activation slice
    static constexpr int STAGE = WBYTES + ABYTES;
    static constexpr int DMA_PER_STAGE = (BN / 16) / 8 + (BM / 8) / 8;   // per wave
};

// Scale buffer of one 4-step chunk: MXFP4 e8m0 dwords (256 B per tile, lane
// order, BN/128 copies per wave), or int4 row scales (128 B per tile = 4 steps
// x 16 fp16 in lane-group order [row / 4][step][row % 4], one 256-byte copy
// per wave: wave w's 256 bytes hold the records
// of tiles (BN/128) w and (BN/128) w + 1 -- for BN = 128 the second half holds
// the next tile's record and is not read), or the int4 records with zero
// points (256 B per tile, copied as the MXFP4 ones).
template <int WF> constexpr bool kRec256 = WF == kWMx || WF == kWI4Z || WF == kWI5;
// int5 adds, per chunk, the fifth-bit planes of the panel's tiles (1 KiB per
// tile: [lane][step] words) and the activation sums of the tile's rows (16 B
// per row: [row][step], at least 128 rows so that every wave copies alike)
template <int BM> constexpr int kI5SumRows = BM > 128 ? BM : 128;
template <int BN, int WF, int BM = 0>
struct PfScales {
    static constexpr int REC = kRec256<WF> ? BN / 16 * 256 : 8 * 256;
    static constexpr int PLANES = WF == kWI5 ? BN / 16 * 1024 : 0;
    static constexpr int SUMS = WF == kWI5 ? kI5SumRows<BM> * 16 : 0;
    static constexpr int BYTES = REC + PLANES + SUMS;
    static constexpr int DMA = (kRec256<WF> ? (BN / 16) / 8 : 1) +
                               (WF == kWI5 ? (BN / 16) / 8 + kI5SumRows<BM> / 128 : 0);   // per wave, per chunk
    static constexpr int TILE_BYTES = kRec256<WF> ? 256 : 128;           // per tile and chunk in HBM
};

// a lane's scale data of step s for weight tile b (0 <= b < BN/16) of the panel
template <int BN, int WF>
__device__ __forceinline__ typename WStep<WF>::T pf_scale(const uint8_t* sbuf, int b, int s, int lane) {
    if constexpr (WF == kWMx) {
        return reinterpret_cast<const uint32_t*>(sbuf)[64 * b + lane] >> (8 * (s & 3));
    } else {
        constexpr int TPW = BN / 128;   // tiles per wave record
        return *reinterpret_cast<const uint2*>(sbuf + 256 * (b / TPW) + 128 * (b % TPW) + 32 * (lane >> 4) +
                                               8 * (s & 3));
    }
}

// the same, split into the LDS read (MXFP4: the whole chunk dword) and the
// selection of step s's byte at the point of use, so that a read issued late
// in a burst does not hold up products that do not need it
template <int BN, int WF>
__device__ __forceinline__ typename WStep<WF>::T pf_scale_raw(const uint8_t* sbuf, int b, int s, int lane) {
    if constexpr (WF == kWMx) return reinterpret_cast<const uint32_t*>(sbuf)[64 * b + lane];
    else return pf_scale<BN, WF>(sbuf, b, s, lane);
}
template <int WF>
__device__ __forceinline__ typename WStep<WF>::T pf_scale_use(typename WStep<WF>::T raw, int s) {
    if constexpr (WF == kWMx) return raw >> (8 * (s & 3));
    else return raw;
}

// Per-workgroup copy sources: one buffer descriptor per operand based at the
// workgroup's tile, per-lane offsets that stay fixed over the K steps (the
// step advance goes into the scalar offset).
template <int BM, int BN>
struct PfSrc {
    i32x4 w, x, sc;
    uint32_t w_off[BN / 128], x_off[BM / 64], s_off[BN / 128];
    i32x4 w5, rs;                       // int5: fifth-bit planes, activation sums
    uint32_t p_off[BN / 128], r_off[2], r_chunk;
};

template <int BM, int BN, int WF>
__device__ __forceinline__ void pf_sources(const PfArgs& a, int tm, int tn, int wave, int lane, PfSrc<BM, BN>& src) {
    const int t0 = tn * (BN / 16);
    const int64_t wblk = (int64_t)a.s_pad * 1024, sblk = (int64_t)a.c_pad * PfScales<BN, WF>::TILE_BYTES;
    src.w = make_rsrc(a.wt + t0 * wblk, (uint64_t)(a.tiles16 - t0) * wblk);
    src.sc = make_rsrc(a.st + t0 * sblk, (uint64_t)(a.tiles16 - t0) * sblk);
    src.x = make_rsrc(a.x8 + (int64_t)tm * BM * a.K, (uint64_t)(a.M - tm * BM) * a.K);
#pragma unroll
    for (int i = 0; i < BN / 128; ++i) {
        // weight (and MXFP4 e8m0) blocks b = wave + 8 i of the BN/16 tiles (clamped to the last tile)
        const int t = min(t0 + wave + 8 * i, a.tiles16 - 1) - t0;
        src.w_off[i] = (uint32_t)(t * wblk) + 16u * lane;
        src.s_off[i] = (uint32_t)(t * sblk) + 4u * lane;
    }
    if constexpr (WF == kWI5) {
        // planes: 4 steps x 256 B per tile and chunk, tile wave + 8 i as the
        // weight blocks; sums: rows tm BM .. of each chunk's [M][4] block, 256
        // bytes per copy (rows past M read the next rows or, past the end, zero)
        src.w5 = make_rsrc(a.w5 + (int64_t)t0 * a.s_pad * 64, (uint64_t)(a.tiles16 - t0) * a.s_pad * 256);
        // (the workspace holds 4 KiB past the last chunk: every copy stays in it)
        const int64_t rs_bytes = (int64_t)a.c_pad * a.M * 16 + 4096;
        src.rs = make_rsrc(a.rs + (int64_t)tm * BM * 4, (uint64_t)(rs_bytes - (int64_t)tm * BM * 16));
        src.r_chunk = (uint32_t)a.M * 16u;
#pragma unroll
        for (int i = 0; i < BN / 128; ++i) {
            const int t = min(t0 + wave + 8 * i, a.tiles16 - 1) - t0;
            src.p_off[i] = (uint32_t)(t * (int64_t)a.s_pad * 256) + 16u * lane;
        }
#pragma unroll
        for (int i = 0; i < kI5SumRows<BM> / 128; ++i) src.r_off[i] = 256u * (wave + 8 * i) + 4u * lane;
    }
    if constexpr (WF == kWI4) {
        // int4 row-scale records: tile (BN/128) wave + lane / 32, 4 bytes per lane
        const int t = min(t0 + wave * (BN / 128) + (lane >> 5), a.tiles16 - 1) - t0;
        src.s_off[0] = (uint32_t)(t * sblk) + 4u * (lane & 31);
    }
#pragma unroll
    for (int i = 0; i < BM / 64; ++i) {
        // activation rows: 8 per copy, 16-byte chunks XOR-swizzled by row
        const int r = 8 * (wave + 8 * i) + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        const int m = min(tm * BM + r, a.M - 1) - tm * BM;
        src.x_off[i] = (uint32_t)m * (uint32_t)a.K + 16u * c;
    }
}

// Copy j (0 <= j < DMA_PER_STAGE) of this wave for K step s into `stage`:
// BN/128 weight blocks, then BM/64 activation row groups.
template <int BM, int BN, int J>
__device__ __forceinline__ void pf_issue_one(const PfSrc<BM, BN>& src, uint8_t* stage, int s, int wave) {
    using S = PfShape<BM, BN>;
    if constexpr (J < BN / 128) {
        lds_dma16(src.w, src.w_off[J], 1024u * s, lds_addr(stage + 1024 * (wave + 8 * J)));
    } else {
        constexpr int i = J - BN / 128;
        lds_dma16(src.x, src.x_off[i], 128u * s, lds_addr(stage + S::WBYTES + 1024 * (wave + 8 * i)));
    }
}

// e8m0 dwords of 4-step chunk c (two 256-byte blocks per wave) into `sbuf`
// (int5: then the planes and the activation sums)
template <int BM, int BN, int WF>
__device__ __forceinline__ void pf_issue_scales(const PfSrc<BM, BN>& src, uint8_t* sbuf, int c, int wave) {
    if constexpr (kRec256<WF>) {
#pragma unroll
        for (int i = 0; i < (BN / 16) / 8; ++i)
            lds_dma4(src.sc, src.s_off[i], 256u * c, lds_addr(sbuf + 256 * (wave + 8 * i)));
        if constexpr (WF == kWI5) {
            using SC = PfScales<BN, WF, BM>;
#pragma unroll
            for (int i = 0; i < (BN / 16) / 8; ++i)
                lds_dma16(src.w5, src.p_off[i], 1024u * c, lds_addr(sbuf + SC::REC + 1024 * (wave + 8 * i)));
#pragma unroll
            for (int i = 0; i < kI5SumRows<BM> / 128; ++i)
                lds_dma4(src.rs, src.r_off[i], src.r_chunk * c, lds_addr(sbuf + SC::REC + SC::PLANES + 256 * (wave + 8 * i)));
        }
    } else {
        lds_dma4(src.sc, src.s_off[0], 128u * c, lds_addr(sbuf + 256 * wave));
    }
}

// copies [J0, J1) of the stage
template <int BM, int BN, int J0, int J1>
__device__ __forceinline__ void pf_issue_range(const PfSrc<BM, BN>& src, uint8_t* stage, int s, int wave) {
    if constexpr (J0 < J1) {
        pf_issue_one<BM, BN, J0>(src, stage, s, wave);
        pf_issue_range<BM, BN, J0 + 1, J1>(src, stage, s, wave);
    }
}

template <int BM, int BN>
__device__ __forceinline__ void pf_issue(const PfSrc<BM, BN>& src, uint8_t* stage, int s, int wave) {
    pf_issue_range<BM, BN, 0, PfShape<BM, BN>::DMA_PER_STAGE>(src, stage, s, wave);
}

// The epilogue's kernel arguments, consumed here so that their scalar loads
// complete before the main loop: an outstanding scalar load makes the LDS
// counter unordered, and the loop's first LDS wait would then be a full
// lgkmcnt(0) on every step instead of a wait for the reads it needs.
__device__ __forceinline__ void pf_args_ready(const PfArgs& a) {
    asm volatile("" ::"s"(a.xs), "s"(a.out), "s"(a.partials), "s"(a.M), "s"(a.N), "s"(a.ks));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    // s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt at their maxima)
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Products of one K step from `st`, with the copies of a later step into
// `nxt` spread between the MFMA groups: a wave whose copy issue stalls on a
// full memory queue then still has products in flight.  The order is pinned
// with scheduling barriers (the scheduler would otherwise sink the products
// below every copy).
template <int BM, int BN, int F>
__device__ __forceinline__ void pf_copies_at(const PfSrc<BM, BN>& src, uint8_t* nxt, int s_nxt, int wave) {
    constexpr int D = PfShape<BM, BN>::DMA_PER_STAGE, FN = PfShape<BM, BN>::FN;
    pf_issue_range<BM, BN, F * D / FN, (F + 1) * D / FN>(src, nxt, s_nxt, wave);
}

template <int BM, int BN, int WF, int F>
__device__ __forceinline__ void pf_group(const uint8_t* wp, const uint8_t* sbuf, int s, int wn, int lane,
                                         const v8i (&bx)[PfShape<BM, BN>::FM], uint4 wa0,
                                         typename WStep<WF>::T sc0, uint4 wa1, typename WStep<WF>::T sc1,
                                         v4f (&acc)[PfShape<BM, BN>::FN][PfShape<BM, BN>::FM],
                                         const PfSrc<BM, BN>& src, uint8_t* nxt, int s_nxt, int wave) {
    using S = PfShape<BM, BN>;
    if constexpr (F < S::FN) {
        const v8i af = wfrag<WF>(wa0);
        // weight fragment F + 2 (and its scale) read two groups ahead
        uint4 wa2 = wa1;
        typename WStep<WF>::T sc2 = sc1;
        if constexpr (F + 2 < S::FN) {
            sc2 = pf_scale_raw<BN, WF>(sbuf, wn * S::FN + F + 2, s, lane);
            wa2 = *reinterpret_cast<const uint4*>(wp + 1024 * (F + 2));
        }
        pf_copies_at<BM, BN, F>(src, nxt, s_nxt, wave);
        const typename WStep<WF>::T scf = pf_scale_use<WF>(sc0, s);
#pragma unroll
        for (int h = 0; h < S::FM; ++h) acc[F][h] = wmma<WF, 0>(af, bx[h], acc[F][h], scf);
        __builtin_amdgcn_sched_barrier(0);
        pf_group<BM, BN, WF, F + 1>(wp, sbuf, s, wn, lane, bx, wa1, sc1, wa2, sc2, acc, src, nxt, s_nxt, wave);
    }
}

template <int BM, int BN, int WF>
__device__ __forceinline__ void pf_compute(const uint8_t* st, int s, int wn, int wm, int lane,
                                           v4f (&acc)[PfShape<BM, BN>::FN][PfShape<BM, BN>::FM],
                                           const uint8_t* sbuf,
                                           const PfSrc<BM, BN>& src, uint8_t* nxt, int s_nxt, int wave) {
    using S = PfShape<BM, BN>;
    const int g = lane >> 4;
    const uint8_t* ws = st;
    const uint8_t* as = st + S::WBYTES;
    const uint8_t* wp = ws + 1024 * (wn * S::FN) + 16 * lane;
    // LDS reads in the order the products need them: all waves leave the
    // barrier together and queue their reads on the LDS at once, so the first
    // product waits only for the first weight fragment, its scale and the first
    // activation fragment; then the other activation fragments and the second
    // weight fragment.  Each group then reads the weight fragment two groups on.
    v8i bx[S::FM];
    const uint4 wa0 = *reinterpret_cast<const uint4*>(wp);
    const typename WStep<WF>::T sc0 = pf_scale_raw<BN, WF>(sbuf, wn * S::FN, s, lane);
    {
        const int r = wm * 16 * S::FM + (lane & 15);
        bx[0] = act_frag<WF>(as + 128 * r, g, (r >> 1) & 7);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 1; h < S::FM; ++h) {
        const int r = wm * 16 * S::FM + 16 * h + (lane & 15);
        bx[h] = act_frag<WF>(as + 128 * r, g, (r >> 1) & 7);
    }
    uint4 wa1 = wa0;
    typename WStep<WF>::T sc1 = sc0;
    if constexpr (S::FN > 1) {
        wa1 = *reinterpret_cast<const uint4*>(wp + 1024);
        sc1 = pf_scale_raw<BN, WF>(sbuf, wn * S::FN + 1, s, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    pf_group<BM, BN, WF, 0>(wp, sbuf, s, wn, lane, bx, wa0, sc0, wa1, sc1, acc, src, nxt, s_nxt, wave);
}


// Output tile and K split of this workgroup: workgroup ids are dealt
// round-robin over the 8 XCDs, so consecutive tiles go to consecutive ids on
// one XCD; tiles are numbered in groups of group_m M-tiles so that the
// workgroups resident on an XCD share weight and activation panels in its L2;
// the K split is the outermost index.
__device__ __forceinline__ bool pf_tile(const PfArgs& a, int& tm, int& tn, int& split) {
    const int tiles = a.tiles_m * a.tiles_n;
    const int total = tiles * a.ks;
    const int per_xcd = (total + 7) >> 3;
    int T = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (T >= total) return false;
    split = T / tiles;
    T -= split * tiles;
    const int gm = a.group_m;
    const int group = T / (gm * a.tiles_n);
    const int first_m = group * gm;
    const int gsize = min(a.tiles_m - first_m, gm);
    const int rem = T % (gm * a.tiles_n);
    tm = first_m + rem % gsize;
    tn = rem / gsize;
    return true;
}

// int4 products of one K step from `st` (one wave row): the wave's FN weight
// fragments are widened to e4m3 and their fp16 row scales converted once, then
// the FM activation fragments are read one at a time (the next one's LDS read
// issued before the current one's products) with the copies for step s_nxt
// spread between the groups.
template <int BM, int BN, int WF, int H>
__device__ __forceinline__ void pfi_groups(const uint8_t* as, int g, int lane, const v8i (&af)[PfShape<BM, BN, WF>::FN],
                                           const float (&sf)[PfShape<BM, BN, WF>::FN][4], v8i bx,
                                           v4f (&acc)[PfShape<BM, BN, WF>::FN][PfShape<BM, BN, WF>::FM],
                                           const PfSrc<BM, BN>& src, uint8_t* nxt, int s_nxt, int wave) {
    using W = PfShape<BM, BN, WF>;
    if constexpr (H < W::FM) {
        constexpr int D = W::DMA_PER_STAGE;
        v8i bn = bx;
        if constexpr (H + 1 < W::FM) {
            const int r = 16 * (H + 1) + (lane & 15);
            bn = act_frag<WF>(as + 128 * r, g, (r >> 1) & 7);
        }
        pf_issue_range<BM, BN, H * D / W::FM, (H + 1) * D / W::FM>(src, nxt, s_nxt, wave);
#pragma unroll
        for (int f = 0; f < W::FN; ++f) {
            const v4f t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[f], bx, v4f{0.f, 0.f, 0.f, 0.f},
                                                                           kFmtFp8, kFmtFp8, 0, kUnitScale, 0,
                                                                           kUnitScale);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[f][H][i] = __builtin_fmaf(sf[f][i], t[i], acc[f][H][i]);
        }
        __builtin_amdgcn_sched_barrier(0);
        pfi_groups<BM, BN, WF, H + 1>(as, g, lane, af, sf, bn, acc, src, nxt, s_nxt, wave);
    }
}

// e4m3 of an integer in [-16, 16] (exact: at most four significant bits)
__device__ __forceinline__ uint32_t e4m3_small_int(int v) {
    if (v == 0) return 0u;
    const uint32_t a = (uint32_t)(v < 0 ? -v : v);
    const int e = 31 - __builtin_clz(a);
    const uint32_t mant = (e >= 3 ? a >> (e - 3) : a << (3 - e)) & 7u;
    return (v < 0 ? 0x80u : 0u) | ((uint32_t)(e + 7) << 3) | mant;
}

// kWI4Z's 16 tables of 16 bytes at zt: table z - 1 holds e4m3(c - z) for
// c = 0..15; one word per thread of the first 64
__device__ __forceinline__ void pfi_fill_zero_tables(uint8_t* zt) {
    const int t = threadIdx.x;
    if (t < 64) {
        const int z = t / 4 + 1, c0 = 4 * (t % 4);
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) w |= e4m3_small_int(c0 + i - z) << (8 * i);
        reinterpret_cast<uint32_t*>(zt)[t] = w;
    }
}

template <int N>
__device__ __forceinline__ uint32_t shl_signed(uint32_t x) {
    if constexpr (N >= 0) return x << N;
    else return x >> (-N);
}
// Word I of a lane's int5 codes: eight low nibbles (nibble j = code 8 I + j)
// and the plane word P (bit 8 q + 2 I + p = fifth bit of code 8 I + 2 q + p)
// -> eight e4m3 bytes of c - 16 in code order.  By (fifth bit, bit 3) the
// values are -16..-9, -8..-1, 0..7, 8..15: four 8-byte tables over c & 7,
// then two byte selects.
template <int I>
__device__ __forceinline__ uint2 int5x8_to_e4m3(uint32_t w, uint32_t P) {
    constexpr uint32_t kA0 = 0xD5D6D7D8u, kA1 = 0xD1D2D3D4u;   // -16 -15 -14 -13 | -12 -11 -10 -9
    constexpr uint32_t kB0 = 0xCACCCED0u, kB1 = 0xB8C0C4C8u;   //  -8  -7  -6  -5 |  -4  -3  -2 -1
    constexpr uint32_t kC0 = 0x44403800u, kC1 = 0x4E4C4A48u;   //   0   1   2   3 |   4   5   6  7
    constexpr uint32_t kD0 = 0x53525150u, kD1 = 0x57565554u;   //   8   9  10  11 |  12  13  14 15
    const uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
    const uint32_t se = ev & 0x07070707u, so = od & 0x07070707u;
    const uint32_t me = ((ev >> 1) & 0x04040404u) | 0x03020100u;
    const uint32_t mo = ((od >> 1) & 0x04040404u) | 0x03020100u;
    const uint32_t fe = (shl_signed<2 - 2 * I>(P) & 0x04040404u) | 0x03020100u;
    const uint32_t fo = (shl_signed<1 - 2 * I>(P) & 0x04040404u) | 0x03020100u;
    const uint32_t e0 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(kB1, kB0, se), __builtin_amdgcn_perm(kA1, kA0, se), me);
    const uint32_t e1 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(kD1, kD0, se), __builtin_amdgcn_perm(kC1, kC0, se), me);
    const uint32_t o0 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(kB1, kB0, so), __builtin_amdgcn_perm(kA1, kA0, so), mo);
    const uint32_t o1 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(kD1, kD0, so), __builtin_amdgcn_perm(kC1, kC0, so), mo);
    const uint32_t e = __builtin_amdgcn_perm(e1, e0, fe);
    const uint32_t o = __builtin_amdgcn_perm(o1, o0, fo);
    return make_uint2(__builtin_amdgcn_perm(o, e, 0x05010400u), __builtin_amdgcn_perm(o, e, 0x07030602u));
}

// int5, first step of a chunk: acc += s (16 - z) x sum(x) over the chunk's
// four steps, one fp32 16x16x4 product per output tile: A = the lane's
// (row lane % 16, step lane / 16) factor from the tile's record, B = the
// activation sum of (token lane % 16, step lane / 16)
template <int BM, int BN>
__device__ __forceinline__ void pfi_zero_fold(const uint8_t* sbuf, int wn, int lane,
                                              v4f (&acc)[PfShape<BM, BN, kWI5>::FN][PfShape<BM, BN, kWI5>::FM]) {
    using W = PfShape<BM, BN, kWI5>;
    using SC = PfScales<BN, kWI5, BM>;
    const int r = lane & 15, u = lane >> 4;
    float zs[W::FN];
#pragma unroll
    for (int f = 0; f < W::FN; ++f) {
        const uint8_t* rec = sbuf + 256 * (wn * W::FN + f);
        const int e = 16 * (r >> 2) + 4 * u + (r & 3);      // lane-group order
        const uint32_t h = *reinterpret_cast<const uint16_t*>(rec + 2 * e);
        zs[f] = f16_to_f32(h) * (float)(int)(int8_t)rec[128 + e];
    }
    const float* sums = reinterpret_cast<const float*>(sbuf + SC::REC + SC::PLANES);
#pragma unroll
    for (int h = 0; h < W::FM; ++h) {
        const float x = sums[4 * (16 * h + r) + u];
#pragma unroll
        for (int f = 0; f < W::FN; ++f) acc[f][h] = __builtin_amdgcn_mfma_f32_16x16x4f32(zs[f], x, acc[f][h], 0, 0, 0);
    }
}

// (zt: kWI4Z's 16 tables of 16 bytes, table z - 1 = e4m3(c - z) for c = 0..15)
template <int BM, int BN, int WF>
__device__ __forceinline__ void pfi_compute(const uint8_t* st, int s, int wn, int lane,
                                            v4f (&acc)[PfShape<BM, BN, WF>::FN][PfShape<BM, BN, WF>::FM],
                                            const uint8_t* sbuf, const PfSrc<BM, BN>& src, uint8_t* nxt, int s_nxt,
                                            int wave, const uint8_t* zt) {
    using W = PfShape<BM, BN, WF>;
    const int g = lane >> 4;
    const uint8_t* as = st + W::WBYTES;
    const uint8_t* wp = st + 1024 * (wn * W::FN) + 16 * lane;
    uint4 q[W::FN];
    uint2 sc[W::FN];
    [[maybe_unused]] uint4 tz[W::FN];
    [[maybe_unused]] uint32_t pl[W::FN];
#pragma unroll
    for (int f = 0; f < W::FN; ++f) {
        q[f] = *reinterpret_cast<const uint4*>(wp + 1024 * f);
        if constexpr (WF == kWI5) {
            // record of tile b (scales as kWI4Z's); the lane's plane word of step s
            sc[f] = *reinterpret_cast<const uint2*>(sbuf + 256 * (wn * W::FN + f) + 32 * g + 8 * (s & 3));
            pl[f] = *reinterpret_cast<const uint32_t*>(sbuf + PfScales<BN, kWI5, BM>::REC + 1024 * (wn * W::FN + f) +
                                                       16 * lane + 4 * (s & 3));
        } else if constexpr (WF == kWI4Z) {
            // record of tile b: scales of the lane's output rows; the zero
            // byte 16 - z of its weight-operand row (row lane % 16) picks the
            // table z - 1
            const uint8_t* rec = sbuf + 256 * (wn * W::FN + f);
            sc[f] = *reinterpret_cast<const uint2*>(rec + 32 * g + 8 * (s & 3));
            const int r = lane & 15;
            const uint32_t zb = rec[128 + 16 * (r >> 2) + 4 * (s & 3) + (r & 3)];
            tz[f] = *reinterpret_cast<const uint4*>(zt + 16 * ((15u - zb) & 15u));
        } else {
            sc[f] = pf_scale<BN, kWI4>(sbuf, wn * W::FN + f, s, lane);
        }
    }
    const int r0 = lane & 15;
    const v8i bx = act_frag<WF>(as + 128 * r0, g, (r0 >> 1) & 7);
    v8i af[W::FN];
    float sf[W::FN][4];
#pragma unroll
    for (int f = 0; f < W::FN; ++f) {
        if constexpr (WF == kWI5) {
            const uint2 a0 = int5x8_to_e4m3<0>(q[f].x, pl[f]), a1 = int5x8_to_e4m3<1>(q[f].y, pl[f]);
            const uint2 a2 = int5x8_to_e4m3<2>(q[f].z, pl[f]), a3 = int5x8_to_e4m3<3>(q[f].w, pl[f]);
            af[f] = v8i{(int)a0.x, (int)a0.y, (int)a1.x, (int)a1.y, (int)a2.x, (int)a2.y, (int)a3.x, (int)a3.y};
        } else if constexpr (WF == kWI4Z) {
            const uint4 qq = q[f], t = tz[f];
            const uint2 a0 = int4x8_to_e4m3_tab(qq.x, t.x, t.y, t.z, t.w);
            const uint2 a1 = int4x8_to_e4m3_tab(qq.y, t.x, t.y, t.z, t.w);
            const uint2 a2 = int4x8_to_e4m3_tab(qq.z, t.x, t.y, t.z, t.w);
            const uint2 a3 = int4x8_to_e4m3_tab(qq.w, t.x, t.y, t.z, t.w);
            af[f] = v8i{(int)a0.x, (int)a0.y, (int)a1.x, (int)a1.y, (int)a2.x, (int)a2.y, (int)a3.x, (int)a3.y};
        } else {
            af[f] = wfrag<WF>(q[f]);
        }
        sf[f][0] = f16_to_f32(sc[f].x & 0xFFFFu);
        sf[f][1] = f16_to_f32(sc[f].x >> 16);
        sf[f][2] = f16_to_f32(sc[f].y & 0xFFFFu);
        sf[f][3] = f16_to_f32(sc[f].y >> 16);
    }
    if constexpr (WF == kWI5) {
        if ((s & 3) == 0) pfi_zero_fold<BM, BN>(sbuf, wn, lane, acc);
    }
    pfi_groups<BM, BN, WF, 0>(as, g, lane, af, sf, bx, acc, src, nxt, s_nxt, wave);
}

// lane holds rows n0..n0+3 of column m in every 16x16 tile: out = bf16(s_m * acc)
template <int BM, int BN, int WF>
__device__ __forceinline__ void pf_epilogue(const PfArgs& a, int tm, int tn, int split, int wn, int wm, int lane,
                                            const v4f (&acc)[PfShape<BM, BN, WF>::FN][PfShape<BM, BN, WF>::FM]) {
    using S = PfShape<BM, BN, WF>;
    const int g = lane >> 4;
    const bool vec = (a.N & 3) == 0;
    if (a.ks > 1) {
        // this split's fp32 sums; the reduction applies the token scale
        float* part = a.partials + (int64_t)split * a.M * a.N;
#pragma unroll
        for (int h = 0; h < S::FM; ++h) {
            const int m = tm * BM + wm * 16 * S::FM + 16 * h + (lane & 15);
            if (m >= a.M) continue;
#pragma unroll
            for (int f = 0; f < S::FN; ++f) {
                const int n0 = tn * BN + (wn * S::FN + f) * 16 + 4 * g;
                if (n0 >= a.N) continue;
                float* o = part + (int64_t)m * a.N + n0;
                if (vec) {
                    *reinterpret_cast<float4*>(o) = make_float4(acc[f][h][0], acc[f][h][1], acc[f][h][2], acc[f][h][3]);
                } else {
                    for (int r = 0; r < 4; ++r)
                        if (n0 + r < a.N) o[r] = acc[f][h][r];
                }
            }
        }
        return;
    }
#pragma unroll
    for (int h = 0; h < S::FM; ++h) {
        const int m = tm * BM + wm * 16 * S::FM + 16 * h + (lane & 15);
        if (m >= a.M) continue;
        const float sm = a.xs ? a.xs[m] : 1.0f;   // W4A4: no token scale
#pragma unroll
        for (int f = 0; f < S::FN; ++f) {
            const int n0 = tn * BN + (wn * S::FN + f) * 16 + 4 * g;
            if (n0 >= a.N) continue;
            uint16_t* o = a.out + (int64_t)m * a.ldo + n0;
            if (vec) {
                const uint32_t h0 = f32_to_bf16_rne(sm * acc[f][h][0]) | (f32_to_bf16_rne(sm * acc[f][h][1]) << 16);
                const uint32_t h1 = f32_to_bf16_rne(sm * acc[f][h][2]) | (f32_to_bf16_rne(sm * acc[f][h][3]) << 16);
                *reinterpret_cast<uint2*>(o) = make_uint2(h0, h1);
            } else {
                for (int r = 0; r < 4; ++r)
                    if (n0 + r < a.N) o[r] = (uint16_t)f32_to_bf16_rne(sm * acc[f][h][r]);
            }
        }
    }
}

// NS-stage ring, copies issued NS - 1 steps ahead; e8m0 chunks (one per four
// steps) in two buffers of their own (chunk c in buffer c & 1: with NS <= 5,
// chunk c is copied from step 4c - NS + 1 >= 4c - 4 on, after the last use of
// chunk c - 2 at step 4c - 5).  Per step s: wait for the copies of step s
// (those of steps s + 1 .. s + NS - 2 may stay in flight), barrier (stage
// visible to all waves; the stage read in step s - 1 is free), issue the e8m0
// chunk that starts at step u = s + NS - 1 (if any), then compute, with the
// copies for step u into the free stage issued between the products.  In
// issue order the copies of step u are: [e8m0 chunk u/4 if u % 4 == 0 and
// u < s1] [weights, activations (of step min(u, s1 - 1))], where [s0, s1) is
// the workgroup's range of K steps (all of K, or one split of it: fp32
// partials, added and scaled by the reduction kernel).
template <int BM, int BN, int NS, int WF>
__global__ __launch_bounds__(kPfThreads) void pf_kernel(PfArgs a) {
    using S = PfShape<BM, BN>;
    using W = PfShape<BM, BN, WF>;
    using SC = PfScales<BN, WF, BM>;
    static_assert(NS >= 3 && NS <= 5, "ring depth");
    constexpr int D = S::DMA_PER_STAGE, DS = SC::DMA;
    constexpr int LDS = kPfBase + NS * S::STAGE + 2 * SC::BYTES;
    static_assert(LDS <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS];
    int tm, tn, split;
    if (!pf_tile(a, tm, tn, split)) return;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wn = wave % W::NWN, wm = wave / W::NWN;

    v4f acc[W::FN][W::FM];
#pragma unroll
    for (int f = 0; f < W::FN; ++f)
#pragma unroll
        for (int h = 0; h < W::FM; ++h) acc[f][h] = v4f{0.f, 0.f, 0.f, 0.f};

    // this workgroup's K steps [s0, s1) (s0 a multiple of 4: whole scale chunks)
    const int s0 = split * a.s_per, s1 = min(a.K >> 7, s0 + a.s_per);
    uint8_t* const base = lds + kPfBase;
    uint8_t* const sbase = base + NS * S::STAGE;
    if constexpr (WF == kWI4Z) {
        // the zero-point tables in the reserved bytes below the stages, before
        // any copy is in flight (so the barrier waits for nothing else)
        pfi_fill_zero_tables(lds);
        __syncthreads();
    }
    PfSrc<BM, BN> src;
    pf_sources<BM, BN, WF>(a, tm, tn, wave, lane, src);
    // prologue: steps s0 .. s0 + NS - 2 (repeating the last step when the range is shorter)
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) {
        const int u = s0 + i;
        if ((u & 3) == 0 && u < s1) pf_issue_scales<BM, BN, WF>(src, sbase + ((u >> 2) & 1) * SC::BYTES, u >> 2, wave);
        pf_issue<BM, BN>(src, base + i * S::STAGE, min(u, s1 - 1), wave);
    }
    int cur = 0, nxt = (NS - 1) * S::STAGE;   // stage offsets of steps s and s + NS - 1
    pf_args_ready(a);
    for (int s = s0; s < s1; ++s) {
        // opaque to the optimiser: stage addresses are formed per step from a
        // few lane bases and immediate offsets instead of being unrolled and
        // hoisted into dozens of live registers
        asm volatile("" : "+s"(cur), "+s"(nxt));
        // copies allowed in flight: those of steps s + 1 .. s + NS - 2, which
        // include at most one e8m0 chunk (NS - 2 <= 3 consecutive steps)
        bool chunk_ahead = false;
#pragma unroll
        for (int v = 1; v <= NS - 2; ++v) chunk_ahead |= ((s + v) & 3) == 0 && s + v < s1;
        if (chunk_ahead) wait_vmcnt<(NS - 2) * D + DS>();
        else wait_vmcnt<(NS - 2) * D>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");     // no LDS access moves across the barrier
        const int u = s + NS - 1;
        if ((u & 3) == 0 && u < s1) pf_issue_scales<BM, BN, WF>(src, sbase + ((u >> 2) & 1) * SC::BYTES, u >> 2, wave);
        // copies for step u; in the last NS - 1 steps they repeat the last step
        // into the free stage, which is never read again (no branch in the
        // product sequence)
        if constexpr (kWiden<WF>)
            pfi_compute<BM, BN, WF>(base + cur, s, wn, lane, acc, sbase + ((s >> 2) & 1) * SC::BYTES, src, base + nxt,
                                    min(u, s1 - 1), wave, lds);
        else
            pf_compute<BM, BN, WF>(base + cur, s, wn, wm, lane, acc, sbase + ((s >> 2) & 1) * SC::BYTES, src,
                                   base + nxt, min(u, s1 - 1), wave);
        cur = cur == (NS - 1) * S::STAGE ? 0 : cur + S::STAGE;
        nxt = nxt == (NS - 1) * S::STAGE ? 0 : nxt + S::STAGE;
    }
    // the repeated copies of the last steps may still be landing: drain them
    // before the workgroup's LDS is released
    wait_vmcnt<0>();
    pf_epilogue<BM, BN, WF>(a, tm, tn, split, wn, wm, lane, acc);
}

// ---------------------------------------------------------------------------
// Tiled band, short tiles (BM <= 128, decode-sized M): the same stages and
// copies, software-pipelined across steps.  A wave holds two register sets
// of fragments (activations, weights, e8m0 dwords of one step); in iteration
// s it multiplies set s while the barrier for stage s + 1 and the LDS reads of
// set s + 1 happen between its MFMA groups, so neither the barrier nor the
// LDS latency stalls the matrix pipe (with one workgroup per CU at these M,
// nothing else would hide them).
//
// Iteration s: [e8m0 chunk for step u = s + NS - 1] [first half of the MFMA
// groups of step s, the copies for step u into stage (s - 1) % NS between
// them] [wait for the copies of step s + 1; lgkmcnt(0); barrier; LDS reads of
// step s + 1 into the other set] [second half of the MFMA groups].
// Stage (s - 1) % NS is free in iteration s: its reads were issued in
// iteration s - 2 and completed (lgkmcnt(0)) before the barrier of iteration
// s - 1, which every wave has passed.  The waits, barrier and reads run in
// the last iteration too (on a stage holding a repeated step), so the MFMA
// sequence has no branch.
// ---------------------------------------------------------------------------

template <int BM, int BN, int WF>
struct PfFrag {
    v8i bx[PfShape<BM, BN>::FM];
    uint4 af[PfShape<BM, BN>::FN];
    typename WStep<WF>::T sc[PfShape<BM, BN>::FN];     // of the fragments' step
};

template <int BM, int BN, int WF>
__device__ __forceinline__ void pf_read(const uint8_t* st, const uint8_t* sbuf, int s, int wn, int wm, int lane,
                                        PfFrag<BM, BN, WF>& F) {
    using S = PfShape<BM, BN>;
    const int g = lane >> 4;
    const uint8_t* as = st + S::WBYTES;
#pragma unroll
    for (int h = 0; h < S::FM; ++h) {
        const int r = wm * 16 * S::FM + 16 * h + (lane & 15);
        const int sw = (r >> 1) & 7;
        const uint8_t* rowp = as + 128 * r;
        F.bx[h] = act_frag<WF>(rowp, g, sw);
    }
    const uint8_t* wp = st + 1024 * (wn * S::FN) + 16 * lane;
#pragma unroll
    for (int f = 0; f < S::FN; ++f) {
        F.af[f] = *reinterpret_cast<const uint4*>(wp + 1024 * f);
        F.sc[f] = pf_scale<BN, WF>(sbuf, wn * S::FN + f, s, lane);
    }
}

__device__ __forceinline__ void wait_lgkm0() {
    // s_waitcnt lgkmcnt(0), vmcnt and expcnt at their maxima
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
}

template <int BM, int BN, int WF, int F0, int F1>
__device__ __forceinline__ void pfp_groups(const PfFrag<BM, BN, WF>& F, v4f (&acc)[PfShape<BM, BN>::FN][PfShape<BM, BN>::FM],
                                           const PfSrc<BM, BN>& src, uint8_t* tgt, int s_cp, int wave) {
    using S = PfShape<BM, BN>;
    if constexpr (F0 < F1) {
        constexpr int H = S::FN > 1 ? S::FN / 2 : 1, D = S::DMA_PER_STAGE;
        if constexpr (F0 < H) pf_issue_range<BM, BN, F0 * D / H, (F0 + 1) * D / H>(src, tgt, s_cp, wave);
        const v8i af = wfrag<WF>(F.af[F0]);
#pragma unroll
        for (int h = 0; h < S::FM; ++h) acc[F0][h] = wmma<WF, 0>(af, F.bx[h], acc[F0][h], F.sc[F0]);
        __builtin_amdgcn_sched_barrier(0);
        pfp_groups<BM, BN, WF, F0 + 1, F1>(F, acc, src, tgt, s_cp, wave);
    }
}

template <int BM, int BN, int NS, int WF>
__device__ __forceinline__ void pfp_iter(int s, int s_end, const PfFrag<BM, BN, WF>& Fc, PfFrag<BM, BN, WF>& Fn,
                                         v4f (&acc)[PfShape<BM, BN>::FN][PfShape<BM, BN>::FM],
                                         const PfSrc<BM, BN>& src, uint8_t* base, uint8_t* sbase, int& cur,
                                         int wn, int wm, int lane, int wave) {
    using S = PfShape<BM, BN>;
    using SC = PfScales<BN, WF>;
    constexpr int D = S::DMA_PER_STAGE, DS = SC::DMA;
    constexpr int H = S::FN > 1 ? S::FN / 2 : 1;
    constexpr int LAST = (NS - 1) * S::STAGE;
    // opaque to the optimiser (addresses from a few bases plus immediates)
    asm volatile("" : "+s"(cur));
    const int nx = cur == LAST ? 0 : cur + S::STAGE;       // stage of step s + 1
    const int tg = cur == 0 ? LAST : cur - S::STAGE;       // stage (s - 1) % NS: copies for step u
    const int u = s + NS - 1;
    if ((u & 3) == 0 && u < s_end) pf_issue_scales<BM, BN, WF>(src, sbase + ((u >> 2) & 1) * SC::BYTES, u >> 2, wave);
    pfp_groups<BM, BN, WF, 0, H>(Fc, acc, src, base + tg, min(u, s_end - 1), wave);
    // pin the first half's products before the barrier (they touch no memory,
    // so nothing else keeps them there): the matrix pipe works through them
    // while the wave waits
#pragma unroll
    for (int f = 0; f < H; ++f)
#pragma unroll
        for (int h = 0; h < S::FM; ++h) asm volatile("" : "+v"(acc[f][h]));
    // copies allowed in flight: those of steps s + 2 .. s + NS - 1, with at
    // most one e8m0 chunk among them (NS - 2 <= 3 consecutive steps)
    bool chunk_ahead = false;
#pragma unroll
    for (int v = 2; v <= NS - 1; ++v) chunk_ahead |= ((s + v) & 3) == 0 && s + v < s_end;
    if (chunk_ahead) wait_vmcnt<(NS - 2) * D + DS>();
    else wait_vmcnt<(NS - 2) * D>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");     // no LDS access moves across the barrier
    pf_read<BM, BN, WF>(base + nx, sbase + (((s + 1) >> 2) & 1) * SC::BYTES, s + 1, wn, wm, lane, Fn);
    __builtin_amdgcn_sched_barrier(0);
    pfp_groups<BM, BN, WF, H, S::FN>(Fc, acc, src, base + tg, min(u, s_end - 1), wave);
    cur = nx;
}

template <int BM, int BN, int NS, int WF>
__global__ __launch_bounds__(kPfThreads) void pfp_kernel(PfArgs a) {
    using S = PfShape<BM, BN>;
    using SC = PfScales<BN, WF>;
    static_assert(NS >= 3 && NS <= 5, "ring depth");
    static_assert(BM <= 128, "two fragment sets fit in registers for short tiles only");
    static_assert(WF == kWMx, "int4 weights take pf_kernel at every tile height");
    constexpr int D = S::DMA_PER_STAGE, DS = SC::DMA;
    constexpr int LDS = kPfBase + NS * S::STAGE + 2 * SC::BYTES;
    static_assert(LDS <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS];
    int tm, tn, split;
    if (!pf_tile(a, tm, tn, split)) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wn = wave % S::NWN, wm = wave / S::NWN;

    v4f acc[S::FN][S::FM];
#pragma unroll
    for (int f = 0; f < S::FN; ++f)
#pragma unroll
        for (int h = 0; h < S::FM; ++h) acc[f][h] = v4f{0.f, 0.f, 0.f, 0.f};

    // this workgroup's K steps [s0, s1) (s0 a multiple of 4: whole scale chunks)
    const int s0 = split * a.s_per, s1 = min(a.K >> 7, s0 + a.s_per);
    uint8_t* const base = lds + kPfBase;
    uint8_t* const sbase = base + NS * S::STAGE;
    PfSrc<BM, BN> src;
    pf_sources<BM, BN, WF>(a, tm, tn, wave, lane, src);
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) {
        const int u = s0 + i;
        if ((u & 3) == 0 && u < s1) pf_issue_scales<BM, BN, WF>(src, sbase + ((u >> 2) & 1) * SC::BYTES, u >> 2, wave);
        pf_issue<BM, BN>(src, base + i * S::STAGE, min(u, s1 - 1), wave);
    }
    // step s0's copies (steps s0 + 1 .. s0 + NS - 2 may stay in flight), then its fragments
    bool chunk_ahead = false;
#pragma unroll
    for (int v = 1; v <= NS - 2; ++v) chunk_ahead |= ((s0 + v) & 3) == 0 && s0 + v < s1;
    if (chunk_ahead) wait_vmcnt<(NS - 2) * D + DS>();
    else wait_vmcnt<(NS - 2) * D>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    PfFrag<BM, BN, WF> F0, F1;
    pf_args_ready(a);
    pf_read<BM, BN, WF>(base, sbase + ((s0 >> 2) & 1) * SC::BYTES, s0, wn, wm, lane, F0);
    int cur = 0;
    for (int s = s0; s < s1; s += 2) {
        pfp_iter<BM, BN, NS, WF>(s, s1, F0, F1, acc, src, base, sbase, cur, wn, wm, lane, wave);
        if (s + 1 < s1) pfp_iter<BM, BN, NS, WF>(s + 1, s1, F1, F0, acc, src, base, sbase, cur, wn, wm, lane, wave);
    }
    // the repeated copies of the last steps may still be landing: drain them
    // before the workgroup's LDS is released
    wait_vmcnt<0>();
    pf_epilogue<BM, BN, kWMx>(a, tm, tn, split, wn, wm, lane, acc);
}

template <int BM, int BN, int NS, int WF>
hipError_t launch_pfp(const PfArgs& a, hipStream_t stream) {
    const int total = a.tiles_m * a.tiles_n * a.ks;
    const int grid = (total + 7) / 8 * 8;
    hipLaunchKernelGGL((pfp_kernel<BM, BN, NS, WF>), dim3(grid), dim3(kPfThreads), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// W4A4: MXFP4 activations x MXFP4 weights on the fp4 x fp4 block-scaled MFMA
// (twice the fp8 rate).  The tile kernel of the MXFP4 weights with the
// activation operand in e2m1 + e8m0: per stage BN/16 weight blocks and BM
// activation rows of 64 bytes (16-byte chunks XOR-swizzled by (row >> 2) & 3,
// so that the 16 rows of a fragment read fall in distinct bank groups); per
// 4-step chunk the weights' e8m0 dwords and BM x 16 bytes of activation e8m0
// (each row's bytes of the chunk, as stored).  Each product takes both
// scales: the weight's byte (step % 4) of its dword and, for the activation
// column of the lane, the byte (lane / 16) of that row's dword for the step.
// No token scale: the epilogue writes bf16(acc).  Same ring, waits and copy
// interleave as pf_kernel.
// ---------------------------------------------------------------------------

template <int BM, int BN>
struct PaShape {
    static constexpr int NWM = BM >= 256 ? 4 : 2;
    static constexpr int NWN = 8 / NWM;
    static constexpr int FN = BN / (16 * NWN);
    static constexpr int FM = BM / (16 * NWM);
    static constexpr int WBYTES = BN / 16 * 1024;          // weight blocks per stage
    static constexpr int ABYTES = BM * 64;                 // activation rows per stage
    static constexpr int STAGE = WBYTES + ABYTES;
    static constexpr int WCP = BN / 128, ACP = BM / 128;   // 1 KiB copies per wave and step
    static constexpr int DMA_PER_STAGE = WCP + ACP;
    static constexpr int SW = BN / 16 * 256, SA = BM * 16; // scale bytes per chunk
    static constexpr int SBYTES = SW + SA;
    static constexpr int SDMA = (BN / 16) / 8 + BM / 128;  // 256-byte copies per wave and chunk
    static_assert(BM == 128 || BM == 256, "W4A4 tiles are 128 or 256 rows");
    static_assert(BN == 256, "W4A4 tiles are 256 wide");
};

template <int BM, int BN>
struct PaSrc {
    i32x4 w, x, sw, sx;
    uint32_t w_off[BN / 128], x_off[BM / 128], sw_off[BN / 128], sx_off[BM / 128];
};

template <int BM, int BN>
__device__ __forceinline__ void pa_sources(const PfArgs& a, int tm, int tn, int wave, int lane, PaSrc<BM, BN>& src) {
    const int t0 = tn * (BN / 16);
    const int64_t wblk = (int64_t)a.s_pad * 1024, sblk = (int64_t)a.c_pad * 256;
    const int64_t rowb = a.K / 2, srow = a.K / 32;
    src.w = make_rsrc(a.wt + t0 * wblk, (uint64_t)(a.tiles16 - t0) * wblk);
    src.sw = make_rsrc(a.st + t0 * sblk, (uint64_t)(a.tiles16 - t0) * sblk);
    src.x = make_rsrc(a.x8 + (int64_t)tm * BM * rowb, (uint64_t)(a.M - tm * BM) * rowb);
    src.sx = make_rsrc(a.xe + (int64_t)tm * BM * srow, (uint64_t)(a.M - tm * BM) * srow);
#pragma unroll
    for (int i = 0; i < BN / 128; ++i) {
        // weight blocks and e8m0 dwords of tiles wave + 8 i (clamped to the last tile)
        const int t = min(t0 + wave + 8 * i, a.tiles16 - 1) - t0;
        src.w_off[i] = (uint32_t)(t * wblk) + 16u * lane;
        src.sw_off[i] = (uint32_t)(t * sblk) + 4u * lane;
    }
#pragma unroll
    for (int i = 0; i < BM / 128; ++i) {
        // activation rows 16 (wave + 8 i) .. + 15 of the tile, lane -> row
        // lane / 4 and stored chunk position lane % 4 (swizzled); rows past M
        // read row M - 1
        const int r = 16 * (wave + 8 * i) + (lane >> 2);
        const int m = min(tm * BM + r, a.M - 1) - tm * BM;
        const int c = (lane & 3) ^ ((r >> 2) & 3);
        src.x_off[i] = (uint32_t)m * (uint32_t)rowb + 16u * c;
        src.sx_off[i] = (uint32_t)m * (uint32_t)srow + 4u * (lane & 3);
    }
}

template <int BM, int BN, int J>
__device__ __forceinline__ void pa_issue_one(const PaSrc<BM, BN>& src, uint8_t* stage, int s, int wave) {
    using S = PaShape<BM, BN>;
    if constexpr (J < S::WCP) {
        lds_dma16(src.w, src.w_off[J], 1024u * s, lds_addr(stage + 1024 * (wave + 8 * J)));
    } else {
        constexpr int i = J - S::WCP;
        lds_dma16(src.x, src.x_off[i], 64u * s, lds_addr(stage + S::WBYTES + 1024 * (wave + 8 * i)));
    }
}
template <int BM, int BN, int J0, int J1>
__device__ __forceinline__ void pa_issue_range(const PaSrc<BM, BN>& src, uint8_t* stage, int s, int wave) {
    if constexpr (J0 < J1) {
        pa_issue_one<BM, BN, J0>(src, stage, s, wave);
        pa_issue_range<BM, BN, J0 + 1, J1>(src, stage, s, wave);
    }
}
// the weight e8m0 dwords and the activation e8m0 rows of 4-step chunk c
template <int BM, int BN>
__device__ __forceinline__ void pa_issue_scales(const PaSrc<BM, BN>& src, uint8_t* sbuf, int c, int wave) {
    using S = PaShape<BM, BN>;
#pragma unroll
    for (int i = 0; i < (BN / 16) / 8; ++i)
        lds_dma4(src.sw, src.sw_off[i], 256u * c, lds_addr(sbuf + 256 * (wave + 8 * i)));
#pragma unroll
    for (int i = 0; i < BM / 128; ++i)
        lds_dma4(src.sx, src.sx_off[i], 16u * c, lds_addr(sbuf + S::SW + 256 * (wave + 8 * i)));
}

template <int BM, int BN, int F>
__device__ __forceinline__ void pa_group(const uint8_t* wp, const uint8_t* sbuf, int s, int wn, int lane,
                                         const v8i (&bx)[PaShape<BM, BN>::FM],
                                         const uint32_t (&scx)[PaShape<BM, BN>::FM], uint4 wa0, uint32_t sc0,
                                         uint4 wa1, uint32_t sc1,
                                         v4f (&acc)[PaShape<BM, BN>::FN][PaShape<BM, BN>::FM],
                                         const PaSrc<BM, BN>& src, uint8_t* nxt, int s_nxt, int wave) {
    using S = PaShape<BM, BN>;
    if constexpr (F < S::FN) {
        const v8i af = frag_fp4(wa0);
        uint4 wa2 = wa1;
        uint32_t sc2 = sc1;
        if constexpr (F + 2 < S::FN) {
            sc2 = reinterpret_cast<const uint32_t*>(sbuf)[64 * (wn * S::FN + F + 2) + lane];
            wa2 = *reinterpret_cast<const uint4*>(wp + 1024 * (F + 2));
        }
        constexpr int D = S::DMA_PER_STAGE;
        pa_issue_range<BM, BN, F * D / S::FN, (F + 1) * D / S::FN>(src, nxt, s_nxt, wave);
        const int scw = (int)(sc0 >> (8 * (s & 3)));
#pragma unroll
        for (int h = 0; h < S::FM; ++h)
            acc[F][h] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bx[h], acc[F][h], kFmtFp4, kFmtFp4, 0,
                                                                         scw, 0, (int)scx[h]);
        __builtin_amdgcn_sched_barrier(0);
        pa_group<BM, BN, F + 1>(wp, sbuf, s, wn, lane, bx, scx, wa1, sc1, wa2, sc2, acc, src, nxt, s_nxt, wave);
    }
}

template <int BM, int BN>
__device__ __forceinline__ void pa_act(const uint8_t* as, const uint8_t* sbuf, int s, int wm, int h, int lane,
                                       v8i& bx, uint32_t& scx) {
    using S = PaShape<BM, BN>;
    const int g = lane >> 4;
    const int r = wm * 16 * S::FM + 16 * h + (lane & 15);
    bx = frag_fp4(*reinterpret_cast<const uint4*>(as + 64 * r + 16 * (g ^ ((r >> 2) & 3))));
    scx = reinterpret_cast<const uint32_t*>(sbuf + S::SW + 16 * r)[s & 3] >> (8 * g);
}

template <int BM, int BN>
__device__ __forceinline__ void pa_compute(const uint8_t* st, int s, int wn, int wm, int lane,
                                           v4f (&acc)[PaShape<BM, BN>::FN][PaShape<BM, BN>::FM],
                                           const uint8_t* sbuf, const PaSrc<BM, BN>& src, uint8_t* nxt, int s_nxt,
                                           int wave) {
    using S = PaShape<BM, BN>;
    const uint8_t* as = st + S::WBYTES;
    const uint8_t* wp = st + 1024 * (wn * S::FN) + 16 * lane;
    // LDS reads in the order the products need them (as in pf_compute)
    v8i bx[S::FM];
    uint32_t scx[S::FM];
    const uint4 wa0 = *reinterpret_cast<const uint4*>(wp);
    const uint32_t sc0 = reinterpret_cast<const uint32_t*>(sbuf)[64 * (wn * S::FN) + lane];
    pa_act<BM, BN>(as, sbuf, s, wm, 0, lane, bx[0], scx[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 1; h < S::FM; ++h) pa_act<BM, BN>(as, sbuf, s, wm, h, lane, bx[h], scx[h]);
    const uint4 wa1 = *reinterpret_cast<const uint4*>(wp + 1024);
    const uint32_t sc1 = reinterpret_cast<const uint32_t*>(sbuf)[64 * (wn * S::FN + 1) + lane];
    __builtin_amdgcn_sched_barrier(0);
    pa_group<BM, BN, 0>(wp, sbuf, s, wn, lane, bx, scx, wa0, sc0, wa1, sc1, acc, src, nxt, s_nxt, wave);
}

template <int BM, int BN, int NS>
__global__ __launch_bounds__(kPfThreads) void pfa_kernel(PfArgs a) {
    using S = PaShape<BM, BN>;
    static_assert(NS >= 3 && NS <= 5, "ring depth");
    constexpr int D = S::DMA_PER_STAGE, DS = S::SDMA;
    constexpr int LDS = kPfBase + NS * S::STAGE + 2 * S::SBYTES;
    static_assert(LDS <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS];
    int tm, tn, split;
    if (!pf_tile(a, tm, tn, split)) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wn = wave % S::NWN, wm = wave / S::NWN;

    v4f acc[S::FN][S::FM];
#pragma unroll
    for (int f = 0; f < S::FN; ++f)
#pragma unroll
        for (int h = 0; h < S::FM; ++h) acc[f][h] = v4f{0.f, 0.f, 0.f, 0.f};

    const int s0 = split * a.s_per, s1 = min(a.K >> 7, s0 + a.s_per);
    uint8_t* const base = lds + kPfBase;
    uint8_t* const sbase = base + NS * S::STAGE;
    PaSrc<BM, BN> src;
    pa_sources<BM, BN>(a, tm, tn, wave, lane, src);
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) {
        const int u = s0 + i;
        if ((u & 3) == 0 && u < s1) pa_issue_scales<BM, BN>(src, sbase + ((u >> 2) & 1) * S::SBYTES, u >> 2, wave);
        pa_issue_range<BM, BN, 0, D>(src, base + i * S::STAGE, min(u, s1 - 1), wave);
    }
    int cur = 0, nxt = (NS - 1) * S::STAGE;
    pf_args_ready(a);
    for (int s = s0; s < s1; ++s) {
        asm volatile("" : "+s"(cur), "+s"(nxt));
        bool chunk_ahead = false;
#pragma unroll
        for (int v = 1; v <= NS - 2; ++v) chunk_ahead |= ((s + v) & 3) == 0 && s + v < s1;
        if (chunk_ahead) wait_vmcnt<(NS - 2) * D + DS>();
        else wait_vmcnt<(NS - 2) * D>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int u = s + NS - 1;
        if ((u & 3) == 0 && u < s1) pa_issue_scales<BM, BN>(src, sbase + ((u >> 2) & 1) * S::SBYTES, u >> 2, wave);
        pa_compute<BM, BN>(base + cur, s, wn, wm, lane, acc, sbase + ((s >> 2) & 1) * S::SBYTES, src, base + nxt,
                           min(u, s1 - 1), wave);
        cur = cur == (NS - 1) * S::STAGE ? 0 : cur + S::STAGE;
        nxt = nxt == (NS - 1) * S::STAGE ? 0 : nxt + S::STAGE;
    }
    wait_vmcnt<0>();
    pf_epilogue<BM, BN, kWMx>(a, tm, tn, split, wn, wm, lane, acc);
}

template <int BM, int BN, int NS>
hipError_t launch_pfa(const PfArgs& a, hipStream_t stream) {
    const int total = a.tiles_m * a.tiles_n * a.ks;
    const int grid = (total + 7) / 8 * 8;
    hipLaunchKernelGGL((pfa_kernel<BM, BN, NS>), dim3(grid), dim3(kPfThreads), 0, stream, a);
    return hipGetLastError();
}

// int5 tiles' pre-pass: each token's activation sum over each 128-wide K
// step, rs[chunk][m][step % 4] (fp32; steps past K give 0), the B operand
// of the zero-point fold.  One thread per (token, step), 128 codes summed
// in fp32 (the sum needs at most 25 significant bits, so it is exact or
// off by one rounding).
__global__ __launch_bounds__(256) void i5_act_sums_kernel(const uint8_t* __restrict__ x8, int M, int K, int c_pad,
                                                          float* __restrict__ rs) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int s_pad = 4 * c_pad;
    if (i >= (int64_t)M * s_pad) return;
    const int s = (int)(i % s_pad);
    const int64_t m = i / s_pad;
    float acc = 0.f;
    if (s < K / 128) {
        const uint4* p = reinterpret_cast<const uint4*>(x8 + m * K + 128 * (int64_t)s);
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = p[j];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t d[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d[e], 1.0f, false);
                const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d[e], 1.0f, true);
                acc += (lo[0] + lo[1]) + (hi[0] + hi[1]);
            }
        }
    }
    rs[((int64_t)(s >> 2) * M + m) * 4 + (s & 3)] = acc;
}

template <int BM, int BN, int NS, int WF>
hipError_t launch_pf(const PfArgs& a, hipStream_t stream) {
    const int total = a.tiles_m * a.tiles_n * a.ks;
    const int grid = (total + 7) / 8 * 8;
    hipLaunchKernelGGL((pf_kernel<BM, BN, NS, WF>), dim3(grid), dim3(kPfThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

void prepared_sizes(int64_t N, int64_t K, size_t* w_bytes, size_t* s_bytes) {
    const int64_t tiles = (N + 15) / 16;
    const int64_t c_pad = (K / 128 + 3) / 4;
    *w_bytes = (size_t)(tiles * c_pad * 4 * 1024);
    *s_bytes = (size_t)(tiles * c_pad * 256);
}

hipError_t launch_prepare(const uint8_t* wq, const uint8_t* we, int64_t N, int64_t K, uint8_t* wt,
                          uint8_t* st, hipStream_t stream) {
    const int tiles = (int)((N + 15) / 16);
    const int c_pad = (int)((K / 128 + 3) / 4);
    const int64_t nw = (int64_t)tiles * c_pad * 4 * 64, ns = (int64_t)tiles * c_pad * 64;
    hipLaunchKernelGGL(prep_w_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, stream, wq,
                       (int)N, (int)K, tiles, 4 * c_pad, reinterpret_cast<uint4*>(wt), 0u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prep_s_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream, we,
                       (int)N, (int)K, tiles, c_pad, reinterpret_cast<uint32_t*>(st));
    return hipGetLastError();
}

void prepared_i4_sizes(int64_t N, int64_t K, size_t* w_bytes, size_t* s_bytes) {
    const int64_t tiles = (N + 15) / 16;
    const int64_t c_pad = (K / 128 + 3) / 4;
    *w_bytes = (size_t)(tiles * c_pad * 4 * 1024);
    *s_bytes = (size_t)(tiles * c_pad * 128);
}

hipError_t launch_prepare_i4(const int32_t* qkn, const uint16_t* sc, int64_t N, int64_t K, uint8_t* wt,
                             uint8_t* st, hipStream_t stream) {
    const int tiles = (int)((N + 15) / 16);
    const int c_pad = (int)((K / 128 + 3) / 4);
    const int64_t nw = (int64_t)tiles * c_pad * 4 * 64, ns = (int64_t)tiles * c_pad * 64;
    hipLaunchKernelGGL(prep_i4w_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t*>(qkn), (int)N, (int)K, tiles, 4 * c_pad,
                       reinterpret_cast<uint4*>(wt));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prep_i4s_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream, sc,
                       (int)N, (int)K, tiles, c_pad, reinterpret_cast<uint16_t*>(st));
    return hipGetLastError();
}

// the same from the transposed [N, K/8] codes (int4g128 GEMM's layout)
hipError_t launch_prepare_i4_nk(const int32_t* qnk, const uint16_t* sc, int64_t N, int64_t K, uint8_t* wt,
                                uint8_t* st, hipStream_t stream) {
    const int tiles = (int)((N + 15) / 16);
    const int c_pad = (int)((K / 128 + 3) / 4);
    const int64_t nw = (int64_t)tiles * c_pad * 4 * 64, ns = (int64_t)tiles * c_pad * 64;
    hipLaunchKernelGGL(prep_w_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<const uint8_t*>(qnk), (int)N, (int)K, tiles, 4 * c_pad,
                       reinterpret_cast<uint4*>(wt), 0x88888888u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prep_i4s_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream, sc,
                       (int)N, (int)K, tiles, c_pad, reinterpret_cast<uint16_t*>(st));
    return hipGetLastError();
}

void prepared_i4z_sizes(int64_t N, int64_t K, size_t* w_bytes, size_t* s_bytes) {
    const int64_t tiles = (N + 15) / 16;
    const int64_t c_pad = (K / 128 + 3) / 4;
    *w_bytes = (size_t)(tiles * c_pad * 4 * 1024);
    *s_bytes = (size_t)(tiles * c_pad * 256);
}

hipError_t launch_prepare_i4z(const int32_t* qkn, const int32_t* qz, const uint16_t* sc, int64_t N, int64_t K,
                              uint8_t* wt, uint8_t* st, hipStream_t stream) {
    const int tiles = (int)((N + 15) / 16);
    const int c_pad = (int)((K / 128 + 3) / 4);
    const int64_t nw = (int64_t)tiles * c_pad * 4 * 64, ns = (int64_t)tiles * c_pad * 64;
    hipLaunchKernelGGL(prep_i4w_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t*>(qkn), (int)N, (int)K, tiles, 4 * c_pad,
                       reinterpret_cast<uint4*>(wt));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prep_i4zs_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream, sc,
                       reinterpret_cast<const uint32_t*>(qz), (int)N, (int)K, tiles, c_pad, st);
    return hipGetLastError();
}

void prepared_i5_sizes(int64_t N, int64_t K, size_t* w_bytes, size_t* w5_bytes, size_t* s_bytes) {
    const int64_t tiles = (N + 15) / 16;
    const int64_t c_pad = (K / 128 + 3) / 4;
    *w_bytes = (size_t)(tiles * c_pad * 4 * 1024);
    *w5_bytes = (size_t)(tiles * c_pad * 4 * 256);
    *s_bytes = (size_t)(tiles * c_pad * 256);
}

hipError_t launch_prepare_i5(const int32_t* qkn, const int32_t* qhi, const uint8_t* qz, const uint16_t* sc,
                             int64_t N, int64_t K, uint8_t* wt, uint8_t* w5, uint8_t* st, hipStream_t stream) {
    const int tiles = (int)((N + 15) / 16);
    const int c_pad = (int)((K / 128 + 3) / 4);
    const int64_t nw = (int64_t)tiles * c_pad * 4 * 64, ns = (int64_t)tiles * c_pad * 64;
    hipLaunchKernelGGL(prep_i4w_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t*>(qkn), (int)N, (int)K, tiles, 4 * c_pad,
                       reinterpret_cast<uint4*>(wt));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prep_i5b_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t*>(qhi), (int)N, (int)K, tiles, 4 * c_pad,
                       reinterpret_cast<uint32_t*>(w5));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prep_i5s_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream, sc, qz,
                       (int)N, (int)K, tiles, c_pad, st);
    return hipGetLastError();
}

// Decode plan on prepared weights: plan fields rt = tiles per workgroup, kw =
// K parts per tile, ks = K splits across workgroups, s_per = chunks per split,
// u = ring depth.  LDS per activation row: 512 bytes per 4-step chunk and 16
// of padding (fp8), or 256 + 16 per chunk and 32 (W4A4 codes and e8m0).
static int64_t lds_row_chunk(bool a4) { return a4 ? 272 : 512; }
static int64_t lds_row_pad(bool a4) { return a4 ? 32 : 16; }

// Wide MXFP4 layers above 8 rows whose whole activation slice fits LDS: one
// workgroup of 16 waves per 16 tiles, one wave per tile over all of K (gate_up
// M = 12 / 16 / 24: 22.0 / 25.4 / 25.5 us with the shape below or the tiled
// kernel, 20.2 / 20.6 / 21.7 us with it: the slice is staged once per 16 tiles
// instead of once per 3).  Needs 128 or more such workgroups.
static bool wide_sixteen(int64_t M, int64_t N, int64_t K, bool a4, bool int4) {
    const int64_t tiles = (N + 15) / 16, c_pad = (K / 128 + 3) / 4;
    if (a4 || int4 || M <= 8 || M > kPreparedDecodeMaxM || tiles < 16 * 128) return false;
    return M * (c_pad * lds_row_chunk(false) + lds_row_pad(false)) <= 160 * 1024;
}

static void prepared_shape(int64_t M, int64_t N, int64_t K, bool a4, bool int4, int* tw, int* kw, int* ks,
                           int* c_per, bool* lds_bound) {
    const int64_t tiles = (N + 15) / 16;
    const int64_t c_pad = (K / 128 + 3) / 4;
    if (wide_sixteen(M, N, K, a4, int4)) {
        *tw = 16;
        *kw = 1;
        *ks = 1;
        *c_per = (int)c_pad;
        *lds_bound = false;
        return;
    }
    const int64_t act_budget = 80 * 1024;          // activations resident in LDS per workgroup
    // K splits across workgroups only when the activations do not fit
    int64_t c_max = (act_budget / M - lds_row_pad(a4)) / lds_row_chunk(a4);
    if (c_max < 1) c_max = 1;
    int64_t s = (c_pad + c_max - 1) / c_max;
    int64_t cp = (c_pad + s - 1) / s;
    s = (c_pad + cp - 1) / cp;
    const int64_t act = M * (cp * lds_row_chunk(a4) + lds_row_pad(a4));   // LDS bytes of the slice
    const bool narrow = (N + 255) / 256 < 64;
    // tiles per workgroup: 3; 4 above M = 16 (more reuse of the activation
    // slice); 2 on narrow layers whose K is not split (more workgroups on the
    // CUs: 160 instead of 107 on a 5120-row layer)
    int64_t t_w = M > 16 ? 4 : (narrow && s == 1 ? 2 : 3);
    if (t_w > tiles) t_w = tiles;
    // K parts per tile: the most of 4, 2, 1 that keeps the launch at about ten
    // waves per CU (tiles x splits x parts <= 2560).  On wide layers whose
    // activation slice leaves LDS room for two workgroups per CU or fewer,
    // more waves per workgroup: four parts for one 16-row activation tile of
    // fp8 or fp4 (with the small activation batch, so that two such
    // workgroups also fit the registers), else twice the parts
    int64_t k_w = 4;
    while (k_w > 1 && tiles * s * k_w > 2560) k_w /= 2;
    *lds_bound = !narrow && (160 * 1024) / act <= 2 && M <= 16 && !int4;
    if (!narrow && (160 * 1024) / act <= 2) k_w = *lds_bound ? 4 : 2 * k_w;
    if (k_w > 4) k_w = 4;
    if (k_w > cp) k_w = cp;
    if (k_w > 16 / t_w) k_w = 16 / t_w;
    if (k_w < 1) k_w = 1;
    *tw = (int)t_w;
    *kw = (int)k_w;
    *ks = (int)s;
    *c_per = (int)cp;
}

// Decode plan: the shape above; ring depth 2 (with the weight stream loaded
// non-temporally, depth 3 measured 2-4 % slower on every shape it had won
// before: gate_up M = 1 / 4 / 8: 17.6 / 17.6 / 18.4 us at depth 2 against
// 17.9 / 18.1 / 19.1, down_proj M = 1: 11.6 against 12.1, W4A4 alike);
// 4 activation loads per thread and batch when one batch covers
// the workgroup's slice or LDS bounds the workgroups per CU (fewer
// registers, more resident waves), else 8.
// Fitted to a sweep of ring depth x batch x tiles x K parts on gfx950 (graph
// replays over 8 weight copies; gate_up 34816 x 5120 and down_proj 5120 x
// 17408, MXFP4 / int4 / W4A4, M from 1 to 32): 1.9 % above the per-shape best
// on average, against the former fixed plan (one or two tiles per workgroup,
// two or four K parts, depth 3, batches of 8): gate_up M = 1 / 8 / 12: 19.6 /
// 22.1 / 22.8 -> 18.7 / 19.7 / 23.8 us (MXFP4); down_proj M = 1 / 8 / 16:
// 13.5 / 15.7 / 18.3 -> 12.2 / 14.4 / 15.9 us; int4 down_proj M = 1 / 16:
// 14.7 / 19.6 -> 12.8 / 17.0 us.
GemmPlan plan_prepared(int64_t M, int64_t N, int64_t K, int ks_hint, int depth, bool a4, bool int4) {
    GemmPlan p{};
    p.band = 2;
    p.mt = (int)((M + 15) / 16);
    int tw, kw, ks, cp;
    bool lds_bound;
    prepared_shape(M, N, K, a4, int4, &tw, &kw, &ks, &cp, &lds_bound);
    if (ks_hint > 0) {   // tuning: ks_hint encodes kw (K parts per tile)
        kw = ks_hint;
        if (kw * tw > 16) kw = 16 / tw;
        if (kw > cp) kw = cp;
    }
    p.rt = tw;
    p.kw = kw;
    p.u = depth > 0 ? depth : 2;
    const int64_t per_row = (int64_t)cp * 512 / (a4 ? 32 : 16);   // 16-byte activation loads per row
    p.ab = lds_bound || M * per_row <= 4 * 64 * (int64_t)tw * kw ? 4 : 8;
    p.ks = ks;
    p.s_per = cp;
    p.tiles = (N + 15) / 16;
    return p;
}

// An explicit split-K decode plan (tuning sweeps): tw tiles and kw K parts
// per workgroup, ring depth `depth`; K split across workgroups only as far as
// the activation slice needs to fit 160 KB of LDS.
GemmPlan plan_prepared_explicit(int64_t M, int64_t N, int64_t K, int tw, int kw, int depth) {
    GemmPlan p{};
    p.band = 2;
    p.mt = (int)((M + 15) / 16);
    const int64_t c_pad = (K / 128 + 3) / 4;
    int64_t c_max = (160 * 1024 / M - lds_row_pad(false)) / lds_row_chunk(false);
    if (c_max < 1) c_max = 1;
    int64_t s = (c_pad + c_max - 1) / c_max;
    int64_t cp = (c_pad + s - 1) / s;
    s = (c_pad + cp - 1) / cp;
    p.rt = tw;
    p.kw = kw > cp ? (int)cp : kw;
    p.u = depth;
    const int64_t per_row = cp * 512 / 16;
    p.ab = M * per_row <= 4 * 64 * (int64_t)tw * p.kw ? 4 : 8;
    p.ks = (int)s;
    p.s_per = (int)cp;
    p.tiles = (N + 15) / 16;
    return p;
}

size_t prepared_lds_bytes(const GemmPlan& p, int64_t M, bool a4) {
    const size_t act = (size_t)(M * ((int64_t)p.s_per * lds_row_chunk(a4) + lds_row_pad(a4)));
    const size_t red = (size_t)p.kw * p.rt * p.mt * 64 * 16;
    return act > red ? act : red;
}

// Tile shape and K split of the tiled kernels.  Tile height by M (64 / 128 /
// 256), the ring as deep as LDS allows for it (5 / 4 / 3 stages); tile width
// 256, or 128 when 256-wide tiles would leave most CUs idle (decode-sized M
// on narrow layers).  With fewer than 128 tiles K is split across workgroups
// (at most one per CU, whole 4-step scale chunks, at least 8 steps each):
// narrow layers at a few hundred rows otherwise run a handful of workgroups
// through all of K (down_proj M = 128: 67 us unsplit, 28 us split).
// Above 128 rows, MXFP4 takes 256-row tiles when their rounds of workgroups
// over the 256 CUs cost no more, a 256-row tile counted as 1.8 128-row ones
// (measured: gate_up M = 200 / 2048 / 4096 and down_proj M = 2048 favour 256
// rows, gate_up M = 512 and down_proj M = 4096 favour 128, M = 1024 even).
// int4 keeps 256-row tiles down to 128 of them: there each wave widens its
// weight fragments once for 16 activation fragments instead of 8, which
// outweighs idle CUs (down_proj-shaped M = 2048, 160 tiles: 290 us vs 399 us
// with 128-row tiles; M = 256, 20 tiles: 278 vs 129 us).
struct TiledShape {
    int bm, bn, tiles_m, tiles_n, ks, s_per;
};
static void tiled_grid(int64_t M, int64_t N, int bm, TiledShape& t, bool int4) {
    t.bm = bm;
    t.tiles_m = (int)((M + bm - 1) / bm);
    const int64_t wide = (int64_t)t.tiles_m * ((N + 255) / 256);
    // 128 wide when 256-wide tiles would be few.  On the down_proj shape at
    // M = 48 / 64 (64-row tiles, K split): MXFP4 22.7 / 24.2 us with 256-wide
    // tiles, 20.0 / 20.7 with 128-wide ones (twice the workgroups, each
    // splitting K as often); int4 at M = 64 30.3 -> 28.7 us, with zero points
    // 32.0 -> 29.8.  On gate_up the 128-wide tiles were slower (MXFP4 M = 64:
    // 34.5 against 29.8 us).
    (void)int4;
    t.bn = wide >= 64 ? 256 : 128;
    t.tiles_n = (int)((N + t.bn - 1) / t.bn);
}
static int64_t tiled_rounds(const TiledShape& t) {
    const int64_t tiles = (int64_t)t.tiles_m * t.tiles_n;
    return tiles < 128 ? 1 : (tiles + 255) / 256;      // few tiles: K split fills one round
}
// K splits (2-4) for at least 128 tiles of the widening kernels (int4, int5:
// vector-ALU bound, long per workgroup): the count that minimises the rounds
// of workgroups per split over 256 CUs, taken when it cuts them by a fifth
// or more, else 1.  160 tiles: 3 (two rounds of a third each); 320: 4 (five
// rounds of a quarter, against two whole ones).
static int64_t rounds_split(int64_t tiles) {
    const double whole = (double)((tiles + 255) / 256);
    int64_t best = 1;
    double best_cost = whole;
    for (int64_t k = 2; k <= 4; ++k) {
        const double c = (double)((tiles * k + 255) / 256) / (double)k;
        if (c < whole * 0.8 && c < best_cost) {
            best = k;
            best_cost = c;
        }
    }
    return best;
}
static void apply_split(TiledShape& t, int64_t steps, int64_t k) {
    if (k <= 1) return;
    int64_t per = (steps + k - 1) / k;
    per = (per + 3) / 4 * 4;
    k = (steps + per - 1) / per;
    if (k > 1) {
        t.ks = (int)k;
        t.s_per = (int)per;
    }
}

static TiledShape tiled_shape(int64_t M, int64_t N, int64_t K, bool int4, int force_ks = 0) {
    TiledShape t{};
    tiled_grid(M, N, M <= 64 ? 64 : 128, t, int4);
    if (M > 128) {
        TiledShape t256{};
        tiled_grid(M, N, 256, t256, int4);
        const bool take = int4 ? (int64_t)t256.tiles_m * t256.tiles_n >= 128
                               : 9 * tiled_rounds(t256) <= 5 * tiled_rounds(t);
        if (take) t = t256;
    }
    const int64_t tiles = (int64_t)t.tiles_m * t.tiles_n, steps = K / 128;
    t.ks = 1;
    t.s_per = (int)steps;
    if (tiles < 128 && steps >= 16) {
        int64_t k = 256 / tiles;                        // at most one round of workgroups
        int64_t per = (steps + k - 1) / k;
        per = (per + 3) / 4 * 4;
        if (per < 8) per = 8;
        k = (steps + per - 1) / per;
        if (k > 1) {
            t.ks = (int)k;
            t.s_per = (int)per;
        }
    } else if (force_ks > 1) {
        apply_split(t, steps, force_ks);
    } else if (int4 && tiles < 256 && steps >= 48) {
        // int4 tiles that leave CUs idle in their one round (down_proj-shaped
        // M = 2048, 160 tiles: three splits, 306 -> 289 us).  From 256 tiles
        // on the partials outweigh it (M = 4096, 320 tiles, four splits: 3-5 %
        // for a 335 MB workspace), and MXFP4 tiles, bound by their copy
        // feed, lost 10 % at 160 tiles: neither is split.
        apply_split(t, steps, rounds_split(tiles));
    }
    return t;
}

// int5 tiles: 64 rows (M <= 64), 128 (M <= 128), else 256; always 128 wide
// (the chunk's fifth-bit planes and activation sums need LDS beside the
// 256-row stages); K split as tiled_shape does when the tiles are few
static TiledShape i5_tiled_shape(int64_t M, int64_t N, int64_t K) {
    TiledShape t{};
    t.bm = M <= 64 ? 64 : (M <= 128 ? 128 : 256);
    t.bn = 128;
    t.tiles_m = (int)((M + t.bm - 1) / t.bm);
    t.tiles_n = (int)((N + 127) / 128);
    const int64_t tiles = (int64_t)t.tiles_m * t.tiles_n, steps = K / 128;
    t.ks = 1;
    t.s_per = (int)steps;
    if (tiles < 128 && steps >= 16) {
        int64_t k = 256 / tiles;
        int64_t per = (steps + k - 1) / k;
        per = (per + 3) / 4 * 4;
        if (per < 8) per = 8;
        k = (steps + per - 1) / per;
        if (k > 1) {
            t.ks = (int)k;
            t.s_per = (int)per;
        }
    } else if (steps >= 48) {
        // a short last round (down_proj-shaped M = 1024 / 2048: 160 / 320
        // tiles, three / four splits: 249 -> 222 us and 473 -> 404 us)
        apply_split(t, steps, rounds_split(tiles));
    }
    return t;
}
// workspace: the activation sums [c_pad][M][4] fp32 and 4 KiB that the last
// tiles' copies may read past them, then (K split) the counter region and
// the fp32 partials
static size_t i5_sums_bytes(int64_t M, int64_t K) {
    const int64_t c_pad = (K / 128 + 3) / 4;
    return (size_t)((c_pad * M * 16 + 4096 + 255) / 256 * 256);
}
size_t i5_tiled_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const TiledShape t = i5_tiled_shape(M, N, K);
    size_t b = i5_sums_bytes(M, K);
    if (t.ks > 1) b += ws_counter_bytes((N + 15) / 16) + (size_t)t.ks * (size_t)M * (size_t)N * sizeof(float);
    return b;
}
bool i5_tiled_fits(int64_t M, int64_t K) {
    // 32-bit buffer offsets: the activation block of a 256-row tile and the
    // per-chunk offset into the sums
    return K <= kPreparedTiledMaxK && (K / 128 + 3) / 4 * M * 16 + 4096 <= (int64_t)UINT32_MAX;
}

hipError_t launch_prepared_tiled_i5(const uint8_t* x8, const float* xs, const uint8_t* wt, const uint8_t* w5,
                                    const uint8_t* st, uint16_t* out, int64_t M, int64_t N, int64_t K, void* ws,
                                    hipStream_t stream) {
    if (!ws || !i5_tiled_fits(M, K)) return hipErrorInvalidValue;
    PfArgs a{};
    a.x8 = x8; a.xs = xs; a.wt = wt; a.st = st; a.out = out;
    a.w5 = reinterpret_cast<const uint32_t*>(w5);
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.ldo = (int)N;
    a.c_pad = (int)((K / 128 + 3) / 4);
    a.s_pad = 4 * a.c_pad;
    a.tiles16 = (int)((N + 15) / 16);
    a.group_m = 8;
    const TiledShape t = i5_tiled_shape(M, N, K);
    a.tiles_m = t.tiles_m;
    a.tiles_n = t.tiles_n;
    a.ks = t.ks;
    a.s_per = t.s_per;
    if ((int64_t)a.tiles_m * a.tiles_n * a.ks > (int64_t)INT32_MAX - 8) return hipErrorInvalidValue;
    uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
    float* rs = reinterpret_cast<float*>(wsb);
    a.rs = rs;
    if (a.ks > 1) a.partials = reinterpret_cast<float*>(wsb + i5_sums_bytes(M, K) + ws_counter_bytes(a.tiles16));
    const int64_t n_sums = M * a.s_pad;
    hipLaunchKernelGGL(i5_act_sums_kernel, dim3((unsigned)((n_sums + 255) / 256)), dim3(256), 0, stream, x8,
                       (int)M, (int)K, a.c_pad, rs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (t.bm == 64) e = launch_pf<64, 128, 5, kWI5>(a, stream);
    else if (t.bm == 128) e = launch_pf<128, 128, 4, kWI5>(a, stream);
    else if (t.bm == 256) e = launch_pf<256, 128, 3, kWI5>(a, stream);
    else return hipErrorInvalidValue;
    if (e != hipSuccess || a.ks == 1) return e;
    return launch_splitk_reduce(a.partials, xs, M, N, a.ks, out, stream);
}

size_t tiled_workspace_bytes(int64_t M, int64_t N, int64_t K, bool int4, int force_ks) {
    const TiledShape t = tiled_shape(M, N, K, int4, force_ks);
    if (t.ks <= 1) return 0;
    return ws_counter_bytes((N + 15) / 16) + (size_t)t.ks * (size_t)M * (size_t)N * sizeof(float);
}

// Tail columns of the 256 x 256 MXFP4 tiles: when their count leaves the
// last round of workgroups part-empty, the leading columns that make whole
// rounds (four or more) keep the 256 x 256 tiles and the rest take narrower
// tiles in one round of their own (every output is still one tile's full-K
// sum, in the same step order).  gate_up M = 4096: 2176 tiles = 8.5 rounds
// on 256 CUs -> 32768 columns in 8 rounds, then 2048 columns as 256 tiles of
// 256 x 128 (567.5 -> 554.8 us, weights streamed from HBM); M = 2048: 1088
// tiles -> 4 rounds, then 256 tiles of 128 x 128 (313.0 -> 289.7 us).  With
// a single whole round (down_proj M = 4096, 320 tiles -> 256 + 256 tiles of
// 128 x 128) it lost 9 %: the short last round of the single launch runs on
// a quarter of the CUs at a higher clock, and the narrow tiles' copy feed per
// product is twice that of the wide ones.
static int device_cus();
struct PfTail {
    int64_t n_main;   // leading columns on 256 x 256 tiles (a multiple of 256)
    int bm, bn;       // the tail's tile
};
static bool pf_tail(const TiledShape& t, int64_t M, int64_t N, PfTail* r) {
    const int64_t cus = device_cus();
    const int64_t tiles = (int64_t)t.tiles_m * t.tiles_n;
    if (t.bm != 256 || t.bn != 256 || t.ks != 1 || tiles < cus || tiles % cus == 0) return false;
    int64_t g = t.tiles_m, h = cus;   // gcd: the 256-wide column tiles per whole-round block
    while (h) {
        const int64_t q = g % h;
        g = h;
        h = q;
    }
    const int64_t per = cus / g, n_tiles = (N / 256) / per * per;
    if (n_tiles == 0 || n_tiles * 256 >= N || t.tiles_m * n_tiles < 4 * cus) return false;
    const int64_t tail = N - n_tiles * 256;
    r->n_main = n_tiles * 256;
    if (((M + 127) / 128) * ((tail + 127) / 128) <= cus) {
        r->bm = 128;
        r->bn = 128;
    } else if (((M + 255) / 256) * ((tail + 127) / 128) <= cus) {
        r->bm = 256;
        r->bn = 128;
    } else {
        return false;
    }
    return true;
}

hipError_t launch_prepared_tiled(const uint8_t* x8, const float* xs, const uint8_t* wt,
                                 const uint8_t* st, uint16_t* out, int64_t M, int64_t N, int64_t K,
                                 void* ws, hipStream_t stream, bool int4, bool zp, int force_ks) {
    PfArgs a{};
    a.x8 = x8; a.xs = xs; a.wt = wt; a.st = st; a.out = out;
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.ldo = (int)N;
    a.c_pad = (int)((K / 128 + 3) / 4);
    a.s_pad = 4 * a.c_pad;
    a.tiles16 = (int)((N + 15) / 16);
    a.group_m = 8;
    const TiledShape t = tiled_shape(M, N, K, int4, force_ks);
    const int bm = t.bm, bn = t.bn;
    a.tiles_m = t.tiles_m;
    a.tiles_n = t.tiles_n;
    a.ks = t.ks;
    a.s_per = t.s_per;
    if ((int64_t)a.tiles_m * a.tiles_n * a.ks > (int64_t)INT32_MAX - 8) return hipErrorInvalidValue;
    if (a.ks > 1) {
        if (!ws) return hipErrorInvalidValue;
        a.partials = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + ws_counter_bytes(a.tiles16));
    }
    // one kernel per (height, width) that tiled_shape can produce; anything
    // else is refused rather than run with a grid the kernel does not assume
    hipError_t e;
    if (int4 && zp) {
        if (bm == 64 && bn == 256) e = launch_pf<64, 256, 5, kWI4Z>(a, stream);
        else if (bm == 64 && bn == 128) e = launch_pf<64, 128, 5, kWI4Z>(a, stream);
        else if (bm == 128 && bn == 128) e = launch_pf<128, 128, 4, kWI4Z>(a, stream);
        else if (bm == 128 && bn == 256) e = launch_pf<128, 256, 4, kWI4Z>(a, stream);
        else if (bm == 256 && bn == 256) e = launch_pf<256, 256, 3, kWI4Z>(a, stream);
        else return hipErrorInvalidValue;
    } else if (int4) {
        if (bm == 64 && bn == 256) e = launch_pf<64, 256, 5, kWI4>(a, stream);
        else if (bm == 64 && bn == 128) e = launch_pf<64, 128, 5, kWI4>(a, stream);
        else if (bm == 128 && bn == 128) e = launch_pf<128, 128, 4, kWI4>(a, stream);
        else if (bm == 128 && bn == 256) e = launch_pf<128, 256, 4, kWI4>(a, stream);
        else if (bm == 256 && bn == 256) e = launch_pf<256, 256, 3, kWI4>(a, stream);
        else return hipErrorInvalidValue;
    } else {
        PfTail tl{};
        if (force_ks == 0 && pf_tail(t, M, N, &tl)) {
            // the leading columns on whole rounds of 256 x 256 tiles
            PfArgs m = a;
            m.N = (int)tl.n_main;
            m.tiles16 = (int)(tl.n_main / 16);
            m.tiles_n = (int)(tl.n_main / 256);
            e = launch_pf<256, 256, 3, kWMx>(m, stream);
            if (e != hipSuccess) return e;
            // the tail columns: weights, scales and outputs from column n_main on
            PfArgs r = a;
            const int64_t t0 = tl.n_main / 16;
            r.wt = wt + t0 * (int64_t)a.s_pad * 1024;
            r.st = st + t0 * (int64_t)a.c_pad * 256;
            r.out = out + tl.n_main;
            r.N = (int)(N - tl.n_main);
            r.tiles16 = (int)((r.N + 15) / 16);
            r.tiles_m = (int)((M + tl.bm - 1) / tl.bm);
            r.tiles_n = (int)((r.N + tl.bn - 1) / tl.bn);
            if (tl.bm == 128) return launch_pfp<128, 128, 4, kWMx>(r, stream);
            return launch_pf<256, 128, 3, kWMx>(r, stream);
        }
        if (bm == 64 && bn == 256) e = launch_pfp<64, 256, 5, kWMx>(a, stream);
        else if (bm == 64 && bn == 128) e = launch_pfp<64, 128, 4, kWMx>(a, stream);
        else if (bm == 128 && bn == 128) e = launch_pfp<128, 128, 4, kWMx>(a, stream);
        else if (bm == 128 && bn == 256) e = launch_pfp<128, 256, 4, kWMx>(a, stream);
        else if (bm == 256 && bn == 256) e = launch_pf<256, 256, 3, kWMx>(a, stream);
        else return hipErrorInvalidValue;
    }
    if (e != hipSuccess || a.ks == 1) return e;
    return launch_splitk_reduce(a.partials, xs, M, N, a.ks, out, stream);
}

// W4A4 tiles: 128 rows up to M = 128, above that 256 rows by the same rounds
// rule as the MXFP4 tiles; always 256 wide; K split as in tiled_shape when the
// tiles are few (this also serves decode-sized M).
static TiledShape w4a4_shape(int64_t M, int64_t N, int64_t K) {
    auto grid = [&](int bm) {
        TiledShape t{};
        t.bm = bm;
        t.bn = 256;
        t.tiles_m = (int)((M + bm - 1) / bm);
        t.tiles_n = (int)((N + 255) / 256);
        return t;
    };
    TiledShape t = grid(128);
    if (M > 128) {
        const TiledShape t256 = grid(256);
        if (9 * tiled_rounds(t256) <= 5 * tiled_rounds(t)) t = t256;
    }
    const int64_t tiles = (int64_t)t.tiles_m * t.tiles_n, steps = K / 128;
    t.ks = 1;
    t.s_per = (int)steps;
    if (tiles < 128 && steps >= 16) {
        int64_t k = 256 / tiles;
        int64_t per = (steps + k - 1) / k;
        per = (per + 3) / 4 * 4;
        if (per < 8) per = 8;
        k = (steps + per - 1) / per;
        if (k > 1) {
            t.ks = (int)k;
            t.s_per = (int)per;
        }
    }
    return t;
}

bool w4a4_decode_route(int64_t M, int64_t N) {
    // where the spread tiles do not apply: the split-K decode kernel for every
    // M it takes (two 16-row activation tiles): with fp4 activations its LDS
    // reads and products cost half of W4A8's (measured on gfx950, gate_up
    // 34816 x 5120: M = 1 / 12 / 13 / 32: 19.8 / 21.4 / 24.2 / 30.0 us, against
    // 32.5 / 35.2 / 35.2 / 34.3 us in the 128-row tile kernel; the spread tiles
    // 16.5-17.9 us for M = 1-32, 19.2 / 20.0 us at M = 48 / 64)
    (void)N;
    return M <= kPreparedDecodeMaxM;
}

size_t w4a4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (spread_a4_fits(M, N, K)) return 0;
    if (w4a4_decode_route(M, N)) return plan_workspace_bytes(plan_prepared(M, N, K, 0, 0, true, false), M, N);
    const TiledShape t = w4a4_shape(M, N, K);
    if (t.ks <= 1) return 0;
    return ws_counter_bytes((N + 15) / 16) + (size_t)t.ks * (size_t)M * (size_t)N * sizeof(float);
}

static hipError_t launch_w4a4_decode(const uint8_t* x4, const uint8_t* xe, const uint8_t* wt, const uint8_t* st,
                                     uint16_t* out, int64_t M, int64_t N, int64_t K, void* ws,
                                     hipStream_t stream);

hipError_t launch_prepared_w4a4(const uint8_t* x4, const uint8_t* xe, const uint8_t* wt, const uint8_t* st,
                                uint16_t* out, int64_t M, int64_t N, int64_t K, void* ws, hipStream_t stream) {
    if (spread_a4_fits(M, N, K)) return launch_spread_a4(x4, xe, wt, st, out, M, N, K, stream);
    if (w4a4_decode_route(M, N)) return launch_w4a4_decode(x4, xe, wt, st, out, M, N, K, ws, stream);
    PfArgs a{};
    a.x8 = x4; a.xe = xe; a.xs = nullptr; a.wt = wt; a.st = st; a.out = out;
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.ldo = (int)N;
    a.c_pad = (int)((K / 128 + 3) / 4);
    a.s_pad = 4 * a.c_pad;
    a.tiles16 = (int)((N + 15) / 16);
    a.group_m = 8;
    const TiledShape t = w4a4_shape(M, N, K);
    a.tiles_m = t.tiles_m;
    a.tiles_n = t.tiles_n;
    a.ks = t.ks;
    a.s_per = t.s_per;
    if ((int64_t)a.tiles_m * a.tiles_n * a.ks > (int64_t)INT32_MAX - 8) return hipErrorInvalidValue;
    if (a.ks > 1) {
        if (!ws) return hipErrorInvalidValue;
        a.partials = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + ws_counter_bytes(a.tiles16));
    }
    hipError_t e;
    if (t.bm == 128 && t.bn == 256) e = launch_pfa<128, 256, 5>(a, stream);
    else if (t.bm == 256 && t.bn == 256) e = launch_pfa<256, 256, 4>(a, stream);
    else return hipErrorInvalidValue;
    if (e != hipSuccess || a.ks == 1) return e;
    return launch_splitk_reduce(a.partials, nullptr, M, N, a.ks, out, stream);
}

PreparedRoute prepared_route(int64_t M, int64_t N, int64_t K, bool int4) {
    // a layer is narrow when 256-wide tiles of 64 rows give fewer than 64
    // workgroups (three quarters of the CUs idle in the tiled kernel)
    const bool narrow = (N + 255) / 256 < 64;
    // narrow MXFP4 layers from 9 to 40 rows: the register-streamed tiles, K
    // split (down_proj M = 16 / 32: 15.5 / 21.0 us with the split-K decode
    // kernel or the tiled kernel, 14.3 / 16.3 us with them)
    if (narrow && !int4 && M > 8 && M <= 40) return PreparedRoute::DTile;
    // wide MXFP4 layers up to 64 rows: the spread tiles, one workgroup per CU
    // over all of K (gate_up M = 1 / 8 / 16 / 32 / 64: 16.7 / 17.1 / 17.4 /
    // 19.5 / 22.8 us against 17.0 / 18.1 / 20.7 / 26 / 28.9 us with the
    // split-K decode or the tiled kernel)
    if (!int4 && spread_fits(M, N, K)) return PreparedRoute::Spread;
    // int4 (and its zero-point form) on the same wide layers above 8 rows: the
    // spread tiles with the decode kernel's split-code products (gate_up-shaped
    // M = 16 / 32 / 64: 18.3 / 22.6 / 33.8 us against 24.5 / 34.1 / 49.4 us
    // with the split-K decode or the tiled kernel, zero points M = 16 / 64:
    // 20.6 / 37.9 against 25.7 / 54.0 us; M = 1 / 8: 17.7 / 18.0 us against
    // 17.0 / 18.0 us, which keep the decode kernel)
    if (int4 && M > 8 && spread_fits(M, N, K)) return PreparedRoute::Spread;
    if (wide_sixteen(M, N, K, false, int4)) return PreparedRoute::Decode;
    // measured on gfx950 (gate_up 34816 x 5120 wide, down_proj 5120 x 17408
    // narrow), split-K decode kernel against the tiled kernel: narrow layers
    // M = 16 / 32: 15.9 / 20.2 us vs 18.4 / 21.1 us (tiled split in K); int4
    // on wide layers, where the tiled kernel's 64-row tiles widen each weight
    // fragment for only four activation fragments: M = 16 / 24 / 32: 26.6 /
    // 30.9 / 33.5 us vs 49 / 50 / 50 us
    if (narrow || int4) return M <= kPreparedDecodeMaxM ? PreparedRoute::Decode : PreparedRoute::Tiled;
    // wide MXFP4 layers: the decode kernel while the activation slice of all
    // of K fits one workgroup's LDS (a K split adds a reduction pass): gate_up
    // M = 12 / 15: 22.4 / 22.7 us vs 24.5 / 24.7 us tiled; M = 16 (split in
    // two): 25.3 vs 24.5 us
    int tw, kw, ks, cp;
    bool lds_bound;
    prepared_shape(M, N, K, false, false, &tw, &kw, &ks, &cp, &lds_bound);
    return M <= 16 && ks == 1 ? PreparedRoute::Decode : PreparedRoute::Tiled;
}

static PDecArgs pdec_args(const GemmPlan& p, const uint8_t* wt, const uint8_t* st, uint16_t* out, int64_t M,
                          int64_t N, int64_t K, void* ws) {
    PDecArgs a{};
    a.wt = reinterpret_cast<const uint4*>(wt);
    a.st = st;
    a.out = out;
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.c_pad = (int)((K / 128 + 3) / 4);
    a.s_pad = 4 * a.c_pad;
    a.tiles = (int)p.tiles;
    a.tw = p.rt;
    a.kw = p.kw;
    a.groups = (int)((p.tiles + p.rt - 1) / p.rt);
    a.ks = p.ks;
    a.c_per = p.s_per;
    if (p.ks > 1) {
        a.counters = reinterpret_cast<uint32_t*>(ws);
        a.partials = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + ws_counter_bytes(p.tiles));
        a.sk_inplace = sk_inplace_fits(p.ks, M, N) ? 1 : 0;
    }
    return a;
}

// the K split's partials reduced by a separate kernel where the last split
// cannot (more splits than it takes in one batch, or offsets past 32 bits)
static hipError_t pdec_finish(const PDecArgs& a, hipError_t e, const float* xs, hipStream_t stream) {
    if (e != hipSuccess || a.ks == 1 || a.sk_inplace) return e;
    return launch_splitk_reduce(a.partials, xs, a.M, a.N, a.ks, a.out, stream);
}

hipError_t launch_prepared_decode(const GemmPlan& p, const uint8_t* x8, const float* xs,
                                  const uint8_t* wt, const uint8_t* st, uint16_t* out, int64_t M,
                                  int64_t N, int64_t K, void* ws, hipStream_t stream, bool int4, bool zp) {
    if (p.ks > 1 && !ws) return hipErrorInvalidValue;
    PDecArgs a = pdec_args(p, wt, st, out, M, N, K, ws);
    a.x8 = x8; a.xs = xs;
    const size_t lds = prepared_lds_bytes(p, M, false);
    const hipError_t e = int4 ? (zp ? launch_pdec_plan<kWI4Z>(p, a, lds, stream) : launch_pdec_plan<kWI4>(p, a, lds, stream))
                              : launch_pdec_plan<kWMx>(p, a, lds, stream);
    return pdec_finish(a, e, xs, stream);
}

// The fused-quant plan: the decode plan, when K is not split across
// workgroups and the whole bf16 activation slice (M x K/8 items of 16 bytes)
// fits one batch of at most 8 loads per thread (4 where that suffices).  The
// plan itself is kept: more K parts per tile to fit a larger slice add waves
// beyond what stays resident (gate_up M = 4 fused in three rounds: 37 us
// against 23 us for the quant kernel and the GEMM).
bool plan_prepared_fused(int64_t M, int64_t N, int64_t K, bool int4, GemmPlan* out) {
    // (the 16-tile workgroups above 8 rows would each quantize a slice of
    // 9+ rows: thousands of vector instructions per thread before the stream)
    if (M > 8) return false;
    GemmPlan p = plan_prepared(M, N, K, 0, 0, false, int4);
    if (p.ks != 1) return false;
    const int64_t items = M * ((int64_t)p.s_per * 512 / 8), threads = 64 * (int64_t)p.rt * p.kw;
    const int64_t groups = (p.tiles + p.rt - 1) / p.rt;
    // every workgroup quantizes the whole slice (about 25 VALU instructions
    // per value, before its weight stream starts): the 8-load batch only with
    // at most one workgroup per CU (down_proj M = 1: 17.9 us fused vs 19.6 us
    // for quant kernel + GEMM; gate_up M = 2, 726 workgroups: 24.7 vs 22.7 us)
    if (items > 8 * threads || (items > 4 * threads && groups > 256)) return false;
    p.ab = items <= 4 * threads ? 4 : 8;
    // ring depth 3 with the 4-load batch: the deeper weight prefetch hides
    // more of the quantizing prologue (gate_up M = 1: 20.2 -> 19.8 us); the
    // 8-load batch and a 3-deep ring exceed the registers
    p.u = p.ab == 8 ? 2 : 3;
    *out = p;
    return true;
}

hipError_t launch_prepared_linear_fused(const GemmPlan& p, const uint16_t* xb, int64_t ldx, const uint8_t* wt,
                                        const uint8_t* st, uint16_t* out, int64_t M, int64_t N, int64_t K,
                                        uint8_t* x8_out, float* xs_out, hipStream_t stream, bool int4) {
    if (p.ks != 1 || p.mt != 1) return hipErrorInvalidValue;
    PDecArgs a = pdec_args(p, wt, st, out, M, N, K, nullptr);
    a.xb = xb; a.ldx = ldx; a.x8_out = x8_out; a.xs_out = xs_out;
    // the fp8 rows, then one amax word per row; the K-part reduction reuses the start
    const size_t act = prepared_lds_bytes(p, M, false) + 4 * (size_t)M;
    const size_t red = (size_t)p.kw * p.rt * p.mt * 64 * 16;
    const size_t lds = act > red ? act : red;
    return int4 ? launch_pdec_fused<kWI4>(p, a, lds, stream) : launch_pdec_fused<kWMx>(p, a, lds, stream);
}

// int5: the split-K decode kernel on rows [0, M), M <= 32
hipError_t launch_prepared_decode_i5(const uint8_t* x8, const float* xs, const uint8_t* wt, const uint8_t* w5,
                                     const uint8_t* st, uint16_t* out, int64_t M, int64_t N, int64_t K, void* ws,
                                     hipStream_t stream) {
    if (M < 1 || M > kPreparedDecodeMaxM) return hipErrorInvalidValue;
    const GemmPlan p = plan_prepared(M, N, K, 0, 0, false, true);
    if (p.ks > 1 && !ws) return hipErrorInvalidValue;
    PDecArgs a = pdec_args(p, wt, st, out, M, N, K, ws);
    a.x8 = x8; a.xs = xs;
    a.w5 = reinterpret_cast<const uint32_t*>(w5);
    const size_t lds = prepared_lds_bytes(p, M, false);
    const hipError_t e = launch_pdec_plan<kWI5>(p, a, lds, stream);
    return pdec_finish(a, e, xs, stream);
}

// W4A4 decode: the split-K decode kernel on MXFP4 activations (no token
// scale: the split-K reduction takes none either)
static hipError_t launch_w4a4_decode(const uint8_t* x4, const uint8_t* xe, const uint8_t* wt, const uint8_t* st,
                                     uint16_t* out, int64_t M, int64_t N, int64_t K, void* ws,
                                     hipStream_t stream) {
    if (M < 1 || M > kPreparedDecodeMaxM) return hipErrorInvalidValue;
    const GemmPlan p = plan_prepared(M, N, K, 0, 0, true, false);
    if (p.ks > 1 && !ws) return hipErrorInvalidValue;
    PDecArgs a = pdec_args(p, wt, st, out, M, N, K, ws);
    a.x8 = x4; a.xe = xe; a.xs = nullptr;
    const size_t lds = prepared_lds_bytes(p, M, true);
    const hipError_t e = launch_pdec_plan<kWMxA4>(p, a, lds, stream);
    return pdec_finish(a, e, nullptr, stream);
}

// The register-streamed tiles of the DTile route: one tile per wave, eight
// waves, K split so that about one round of workgroups covers the CUs.
DtPlan plan_dtile_route(int64_t M, int64_t N, int64_t K) {
    const int64_t groups = ((N + 15) / 16 + 7) / 8;
    int64_t ks = 256 / groups;
    ks = ks < 1 ? 1 : (ks > 8 ? 8 : ks);
    return plan_dtile(M, N, K, 1, 8, (int)ks);
}

// Register-streamed tiles: R tiles per wave (1, 2 or 4), K split across ks
// workgroups (units of two steps per split rounded up to an even count).
DtPlan plan_dtile(int64_t M, int64_t N, int64_t K, int R, int W, int ks) {
    DtPlan p{};
    p.mt = (int)((M + 15) / 16);
    p.r = R;
    p.w = W;
    const int64_t units = 2 * ((K / 128 + 3) / 4);            // two-step units of the padded steps
    if (ks < 1) ks = 1;
    int64_t per = (units + ks - 1) / ks;
    per = (per + 1) / 2 * 2;
    p.h_per = (int)per;
    p.ks = (int)((units + per - 1) / per);
    p.tiles = (N + 15) / 16;
    p.groups = (p.tiles + W * R - 1) / (W * R);
    return p;
}

size_t dtile_workspace_bytes(const DtPlan& p, int64_t M, int64_t N) {
    if (p.ks <= 1) return 0;
    return ws_counter_bytes(p.tiles) + (size_t)p.ks * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_dtile(const DtPlan& p, const uint8_t* x8, const float* xs, const uint8_t* wt, const uint8_t* st,
                        uint16_t* out, int64_t M, int64_t N, int64_t K, void* ws, hipStream_t stream) {
    if (M < 1 || M > 64 || p.mt != (int)((M + 15) / 16) || K % 128 != 0) return hipErrorInvalidValue;
    if (p.ks > 1 && !ws) return hipErrorInvalidValue;
    if ((int64_t)p.groups * p.ks > (int64_t)INT32_MAX) return hipErrorInvalidValue;
    DtArgs a{};
    a.x8 = x8; a.xs = xs; a.out = out;
    a.wt = reinterpret_cast<const uint4*>(wt);
    a.st = reinterpret_cast<const uint32_t*>(st);
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.c_pad = (int)((K / 128 + 3) / 4);
    a.s_pad = 4 * a.c_pad;
    a.tiles = (int)p.tiles;
    a.groups = (int)p.groups;
    a.ks = p.ks;
    a.h_per = p.h_per;
    if (p.ks > 1) {
        a.counters = reinterpret_cast<uint32_t*>(ws);
        a.partials = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + ws_counter_bytes(p.tiles));
        a.sk_inplace = sk_inplace_fits(p.ks, M, N) ? 1 : 0;
    }
    hipError_t e;
#define W4A8_DT(MT, R, W) else if (p.mt == MT && p.r == R && p.w == W) e = launch_dtile_inst<MT, R, W>(a, stream);
    if (false) e = hipErrorInvalidValue;
    // four tiles per wave only with one or two activation tiles (beyond, the
    // ring and accumulators exceed the registers); 16 waves (128 registers
    // each) with one tile per wave
    W4A8_DT(1, 1, 4) W4A8_DT(1, 2, 4) W4A8_DT(1, 4, 4) W4A8_DT(2, 1, 4) W4A8_DT(2, 2, 4) W4A8_DT(2, 4, 4)
    W4A8_DT(3, 1, 4) W4A8_DT(3, 2, 4) W4A8_DT(4, 1, 4) W4A8_DT(4, 2, 4)
    W4A8_DT(1, 1, 8) W4A8_DT(1, 2, 8) W4A8_DT(2, 1, 8) W4A8_DT(2, 2, 8) W4A8_DT(3, 1, 8) W4A8_DT(4, 1, 8)
    W4A8_DT(4, 2, 8) W4A8_DT(1, 1, 16) W4A8_DT(2, 1, 16) W4A8_DT(3, 1, 16) W4A8_DT(4, 1, 16)
    else return hipErrorInvalidValue;
#undef W4A8_DT
    if (e != hipSuccess || p.ks == 1 || a.sk_inplace) return e;   // else reduced by a second kernel
    return launch_splitk_reduce(a.partials, xs, M, N, p.ks, out, stream);
}


// CUs of the current device (cached per device)
static int device_cus() {
    static int cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// Spread tiles: one workgroup per CU (at most tiles / 8, so that every wave
// has a tile); R = the most tiles a wave gets; ring depth D and the e8m0
// dwords per step or per chunk (CS) as below.
SpPlan plan_spread(int64_t M, int64_t N, int64_t K, int D, int CS) {
    SpPlan p{};
    p.mt = (int)((M + 15) / 16);
    const int64_t s_pad = 4 * ((K / 128 + 3) / 4);
    // default: ring depth 4 with the e8m0 dwords once per chunk where the
    // padded steps are a multiple of 8 (gate_up M = 1 / 8 / 16 / 64: 16.7 /
    // 17.1 / 17.4 / 22.8 us, against 17.4 / 17.7 / 18.2 / 24.4 us with the
    // dwords loaded every step at depth 8 / 8 / 8 / 4)
    p.d = D > 0 ? D : 4;
    p.cs = CS >= 0 ? CS : (p.d == 4 && s_pad % 8 == 0 ? 1 : 0);
    p.tiles = (N + 15) / 16;
    int64_t g = device_cus();
    if (g > p.tiles / kSpWaves) g = p.tiles / kSpWaves;
    p.groups = g;
    p.r = g >= 1 ? (int)(((p.tiles + g - 1) / g + kSpWaves - 1) / kSpWaves) : 0;
    return p;
}

// the output block of a workgroup (M rows, at most ceil(tiles / groups) tiles of
// 32 bytes) assembled in the stage ring for 16-byte row stores
static int spread_out16(const uint16_t* out, int64_t M, int64_t N, const SpPlan& p) {
    const int64_t nt_max = (p.tiles + p.groups - 1) / p.groups;
    return (N % 8 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0 &&
            M * 32 * nt_max <= (int64_t)kSpStages * kSpStage) ? 1 : 0;
}

bool spread_fits(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || M > 64 || K % 128 != 0) return false;
    const SpPlan p = plan_spread(M, N, K, 0, -1);
    // most CUs busy, and an instantiated tile count
    return p.groups * 4 >= (int64_t)device_cus() * 3 && p.r >= 1 && p.r <= 2;
}

// the linear on one bf16 token with its quantization fused into the spread
// tiles: the quantized row resident in LDS (K + 4 bytes of the 32 KiB), K
// steps a multiple of 8 (the trips of two chunks, no padding steps), the row
// read as 16-byte items
bool spread_fq_fits(int64_t M, int64_t N, int64_t K) {
    return M == 1 && spread_fits(M, N, K) && (K / 128) % 8 == 0 && K <= 8192;
}

hipError_t launch_spread_fq(const uint16_t* xb, const uint8_t* wt, const uint8_t* st, uint16_t* out,
                            uint8_t* x8_out, float* xs_out, int64_t N, int64_t K, hipStream_t stream) {
    if (!spread_fq_fits(1, N, K)) return hipErrorInvalidValue;
    const SpPlan p = plan_spread(1, N, K, 0, -1);
    if (p.d != 4 || !p.cs || p.groups < 1 || p.r < 1 || p.r > 2) return hipErrorInvalidValue;
    if (p.tiles < (int64_t)kSpWaves * p.groups || (p.tiles + p.groups - 1) / p.groups > (int64_t)kSpWaves * p.r)
        return hipErrorInvalidValue;
    SpArgs a{};
    a.xb = xb; a.x8_out = x8_out; a.xs_out = xs_out; a.out = out;
    a.wt = reinterpret_cast<const uint4*>(wt);
    a.st = reinterpret_cast<const uint32_t*>(st);
    a.M = 1; a.N = (int)N; a.K = (int)K;
    a.c_pad = (int)((K / 128 + 3) / 4);
    a.s_pad = 4 * a.c_pad;
    a.steps = (int)(K / 128);
    a.tiles = (int)p.tiles;
    a.groups = (int)p.groups;
    a.out16 = spread_out16(out, 1, N, p);
    if (p.r == 1) return launch_spread_inst<1, 1, 4, true, false, true>(a, stream);
    return launch_spread_inst<1, 2, 4, true, false, true>(a, stream);
}

// the spread tiles on the plain layout: K steps a multiple of 8 (no padding
// steps; the e8m0 bytes gathered once per chunk, in trips of two chunks)
bool spread_plain_fits(int64_t M, int64_t N, int64_t K) {
    return spread_fits(M, N, K) && (K / 128) % 8 == 0;
}

hipError_t launch_spread(const SpPlan& p, const uint8_t* x8, const float* xs, const uint8_t* wt, const uint8_t* st,
                         uint16_t* out, int64_t M, int64_t N, int64_t K, hipStream_t stream, bool plain,
                         bool x_step_major) {
    if (M < 1 || M > 64 || p.mt != (int)((M + 15) / 16) || K % 128 != 0 || p.groups < 1) return hipErrorInvalidValue;
    if (p.groups > (int64_t)INT32_MAX || p.tiles > (int64_t)INT32_MAX / 16) return hipErrorInvalidValue;
    // every wave has a tile, and none more than R
    if (p.tiles < (int64_t)kSpWaves * p.groups || (p.tiles + p.groups - 1) / p.groups > (int64_t)kSpWaves * p.r)
        return hipErrorInvalidValue;
    SpArgs a{};
    a.x8 = x8; a.xs = xs; a.out = out;
    a.wt = reinterpret_cast<const uint4*>(wt);
    a.st = reinterpret_cast<const uint32_t*>(st);
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.c_pad = (int)((K / 128 + 3) / 4);
    a.s_pad = 4 * a.c_pad;
    a.steps = (int)(K / 128);
    a.tiles = (int)p.tiles;
    a.groups = (int)p.groups;
    a.out16 = spread_out16(out, M, N, p);
    a.xrs = x_step_major ? 128 : K;
    a.xss = x_step_major ? 128 * M : 128;
    if (a.s_pad % p.d != 0 || (p.cs && (p.d != 4 || a.s_pad % 8 != 0))) return hipErrorInvalidValue;
    if (plain) {
        // [N, K/2] codes and [N, K/32] e8m0 in place of the fragment-order blocks
        if (a.steps % 8 != 0 || p.d != 4 || !p.cs) return hipErrorInvalidValue;
#define W4A8_SPL(MT, R) \
    else if (p.mt == MT && p.r == R) return launch_spread_inst<MT, R, 4, true, true>(a, stream);
        if (false) {}
        W4A8_SPL(1, 1) W4A8_SPL(2, 1) W4A8_SPL(3, 1) W4A8_SPL(4, 1)
        W4A8_SPL(1, 2) W4A8_SPL(2, 2) W4A8_SPL(3, 2) W4A8_SPL(4, 2)
#undef W4A8_SPL
        return hipErrorInvalidValue;
    }
#define W4A8_SP(MT, R, D, CS) \
    else if (p.mt == MT && p.r == R && p.d == D && p.cs == CS) return launch_spread_inst<MT, R, D, CS>(a, stream);
    if (false) {}
    W4A8_SP(1, 1, 4, 0) W4A8_SP(2, 1, 4, 0) W4A8_SP(3, 1, 4, 0) W4A8_SP(4, 1, 4, 0)
    W4A8_SP(1, 2, 4, 0) W4A8_SP(2, 2, 4, 0) W4A8_SP(3, 2, 4, 0) W4A8_SP(4, 2, 4, 0)
    W4A8_SP(1, 1, 4, 1) W4A8_SP(2, 1, 4, 1) W4A8_SP(3, 1, 4, 1) W4A8_SP(4, 1, 4, 1)
    W4A8_SP(1, 2, 4, 1) W4A8_SP(2, 2, 4, 1) W4A8_SP(3, 2, 4, 1) W4A8_SP(4, 2, 4, 1)
    W4A8_SP(1, 1, 8, 0) W4A8_SP(1, 2, 8, 0) W4A8_SP(2, 2, 8, 0) W4A8_SP(3, 2, 8, 0) W4A8_SP(4, 2, 8, 0)
#undef W4A8_SP
    return hipErrorInvalidValue;
}

// W4A4 on the spread tiles: the wide layers of the fp8 form
bool spread_a4_fits(int64_t M, int64_t N, int64_t K) {
    return spread_fits(M, N, K);
}

hipError_t launch_spread_a4(const uint8_t* x4, const uint8_t* xe, const uint8_t* wt, const uint8_t* st,
                            uint16_t* out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    if (!spread_a4_fits(M, N, K)) return hipErrorInvalidValue;
    const SpPlan p = plan_spread(M, N, K, 4, 1);
    if (p.groups < 1 || p.groups > (int64_t)INT32_MAX || p.tiles > (int64_t)INT32_MAX / 16 ||
        p.mt != (int)((M + 15) / 16))
        return hipErrorInvalidValue;
    // every wave has a tile, and none more than R
    if (p.tiles < (int64_t)kSpWaves * p.groups || (p.tiles + p.groups - 1) / p.groups > (int64_t)kSpWaves * p.r)
        return hipErrorInvalidValue;
    SpArgs a{};
    a.x8 = x4; a.xe = xe; a.xs = nullptr; a.out = out;
    a.wt = reinterpret_cast<const uint4*>(wt);
    a.st = reinterpret_cast<const uint32_t*>(st);
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.c_pad = (int)((K / 128 + 3) / 4);
    a.s_pad = 4 * a.c_pad;
    a.steps = (int)(K / 128);
    a.tiles = (int)p.tiles;
    a.groups = (int)p.groups;
    a.out16 = spread_out16(out, M, N, p);
#define W4A8_SA4(MT, R)                                                                                 \
    if (p.mt == MT && p.r == R) {                                                                     \
        hipLaunchKernelGGL((spread_a4_kernel<MT, R>), dim3(a.groups), dim3(kSpThreads), 0, stream, a); \
        return hipGetLastError();                                                                     \
    }
    W4A8_SA4(1, 1) W4A8_SA4(2, 1) W4A8_SA4(3, 1) W4A8_SA4(4, 1)
    W4A8_SA4(1, 2) W4A8_SA4(2, 2) W4A8_SA4(3, 2) W4A8_SA4(4, 2)
#undef W4A8_SA4
    return hipErrorInvalidValue;
}

hipError_t launch_spread_i4(const uint8_t* x8, const float* xs, const uint8_t* wt, const uint8_t* st, uint16_t* out,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream, int wf, const uint8_t* w5) {
    if (wf != kWI4 && wf != kWI4Z && wf != kWI5) return hipErrorInvalidValue;
    if ((wf == kWI5) != (w5 != nullptr)) return hipErrorInvalidValue;
    if (!spread_fits(M, N, K)) return hipErrorInvalidValue;
    const SpPlan p = plan_spread(M, N, K, 4, 1);
    if (p.groups < 1 || p.groups > (int64_t)INT32_MAX || p.tiles > (int64_t)INT32_MAX / 16 ||
        p.mt != (int)((M + 15) / 16))
        return hipErrorInvalidValue;
    // every wave has a tile, and none more than R
    if (p.tiles < (int64_t)kSpWaves * p.groups || (p.tiles + p.groups - 1) / p.groups > (int64_t)kSpWaves * p.r)
        return hipErrorInvalidValue;
    SpArgs a{};
    a.x8 = x8; a.xs = xs; a.out = out;
    a.wt = reinterpret_cast<const uint4*>(wt);
    a.st = reinterpret_cast<const uint32_t*>(st);
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.c_pad = (int)((K / 128 + 3) / 4);
    a.s_pad = 4 * a.c_pad;
    a.steps = (int)(K / 128);
    a.tiles = (int)p.tiles;
    a.groups = (int)p.groups;
    a.out16 = spread_out16(out, M, N, p);
    a.xrs = K;
    a.xss = 128;
    a.w5 = reinterpret_cast<const uint32_t*>(w5);
#define W4A8_SI4(MT, R, WF)                                                                                 \
    if (p.mt == MT && p.r == R && wf == WF) {                                                             \
        hipLaunchKernelGGL((spread_i4_kernel<MT, R, WF>), dim3(a.groups), dim3(kSpThreads), 0, stream, a); \
        return hipGetLastError();                                                                         \
    }
    W4A8_SI4(1, 1, kWI4) W4A8_SI4(2, 1, kWI4) W4A8_SI4(3, 1, kWI4) W4A8_SI4(4, 1, kWI4)
    W4A8_SI4(1, 2, kWI4) W4A8_SI4(2, 2, kWI4) W4A8_SI4(3, 2, kWI4) W4A8_SI4(4, 2, kWI4)
    W4A8_SI4(1, 1, kWI4Z) W4A8_SI4(2, 1, kWI4Z) W4A8_SI4(3, 1, kWI4Z) W4A8_SI4(4, 1, kWI4Z)
    W4A8_SI4(1, 2, kWI4Z) W4A8_SI4(2, 2, kWI4Z) W4A8_SI4(3, 2, kWI4Z) W4A8_SI4(4, 2, kWI4Z)
    W4A8_SI4(1, 1, kWI5) W4A8_SI4(2, 1, kWI5) W4A8_SI4(3, 1, kWI5) W4A8_SI4(4, 1, kWI5)
    W4A8_SI4(1, 2, kWI5) W4A8_SI4(2, 2, kWI5) W4A8_SI4(3, 2, kWI5) W4A8_SI4(4, 2, kWI5)
#undef W4A8_SI4
    return hipErrorInvalidValue;
}

}  // namespace w4a8
