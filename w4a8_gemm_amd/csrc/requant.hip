// requant.hip -- NVFP4 -> MXFP4 requantization on gfx950.
//
// "radiance_nvfp4.py": dequant_nvfp4 (W = e2m1 * e4m3 scale / global divisor),
// _block_exponent (ocp / noclip rules), e2m1_index (nearest grid point, ties to
// the even index, saturating at 6), _encode_blocks (squared error per block),
// quant_mxfp4 (mse picks noclip or noclip-1; sign bit only on nonzero codes;
// e8m0 = e + 127).
//
// The same encoder serves the other load-time inputs of the page's schemes
// (RadianceBf16ToMxfp4: the bf16 weight itself; RadianceFp8ChannelToMxfp4: the
// e4m3 weight times its row's fp32 scale, one rounded product); only the
// stage that forms the block's 32 fp32 values differs.
//
// Mapping: one lane per 32-element block.  A block is 16 bytes of NVFP4 codes and
// 2 e4m3 scale bytes in, 16 bytes of MXFP4 codes and 1 e8m0 byte out, and the
// blocks of a row-major [rows, K] weight are consecutive in all four arrays, so a
// wavefront reads and writes contiguous 1 KiB / 128 B / 1 KiB / 64 B runs.  Each
// workgroup takes a contiguous range of blocks inside one partition (so its
// divisor is uniform) in iterations of one block per lane, the next
// iteration's input loaded before the current one is encoded, so that loads
// stay in flight while the vector ALU works.  One launch covers every
// partition and row chunk of a call.  Squared errors are summed in fp32 in
// element order 0..31, each square rounded first, with no fused multiply-add
// (the file is compiled with -ffp-contract=off), so the mse decision is a fixed
// function of the inputs.
#include "w4a8_internal.h"

#pragma clang fp contract(off)

namespace w4a8 {
namespace {

constexpr int kThreads = 256;

// Block exponent from amax (>= 0), exact integer forms of the closed rules:
//   ocp     floor(log2 a) - 2
//   noclip  the least e with a <= 6 * 2^e
// amax below the smallest normal is raised to it; amax == 0 gives 0; the result
// is clamped to [-127, 127].
__device__ __forceinline__ int block_exponent(float amax, int mode) {
    if (!(amax > 0.0f)) return 0;
    const float safe = fmaxf(amax, 0x1p-126f);
    const uint32_t bits = __float_as_uint(safe);
    const int p = (int)(bits >> 23) - 127;  // floor(log2 safe)
    int e;
    if (mode == W4A8_EXP_OCP)
        e = p - 2;
    else  // mantissa <= 1.5 fits under 6 * 2^(p-2), otherwise one binade up
        e = p - 2 + ((bits & 0x7FFFFFu) > 0x400000u ? 1 : 0);
    return max(-127, min(127, e));
}

// Encode one block at exponent e: the e2m1 codes of w / 2^e and, if ERR, the
// fp32 squared error of the block summed in element order.  The codes come
// from the matrix-format conversion instruction, whose rounding is the page's
// e2m1_index on magnitudes (nearest grid point, ties to the even index -- the
// index's low bit is the mantissa bit -- and values above 6 saturating at 6;
// checked against the rule for every magnitude class on gfx950), with the
// input's sign in bit 3.  A negative value that rounds to zero therefore comes
// out as code 8 (-0), which is folded to code 0: the page sets the sign only on
// nonzero codes.
template <int T>
__device__ __forceinline__ uint32_t to_e2m1(uint32_t old, float a0, float a1) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a0, a1, 1.0f, T);   // byte T <- codes of a0, a1
}
// the sign bit of every nibble whose magnitude bits are zero cleared (8 -> 0)
__device__ __forceinline__ uint32_t fold_neg_zero(uint32_t x) {
    const uint32_t m = x & 0x77777777u;
    const uint32_t nz = (m | (m >> 1) | (m >> 2)) & 0x11111111u;   // nibble bit 0: magnitude != 0
    return m | (x & (nz << 3));
}
// squared errors of the two elements of byte T, added to err in element order.
// The grid value q has the sign of w (or is zero), so q - w = +-(|q| - |w|) and
// its square is that of |q| - |w|: the difference is exact (the magnitudes are
// within a factor of two of each other unless q is 0) and the square rounded
// once, as for q - w.
template <int T>
__device__ __forceinline__ float byte_err(uint32_t codes, const float* w2, float scale, float err) {
    const auto g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, T);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float d = fabsf(g[u]) * scale - fabsf(w2[u]);
        const float sq = d * d;
        err = err + sq;
    }
    return err;
}

template <bool ERR>
__device__ __forceinline__ float encode_block(const float* w, int e, uint32_t* code) {
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, normal for e in [-127, 126]
    const float scale = ldexpf(1.0f, e);                            // 2^e, exact (subnormal at -127)
    float err = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float* b = w + 8 * q;
        // w / 2^e, each product correctly rounded
        uint32_t packed = to_e2m1<0>(0u, b[0] * inv, b[1] * inv);
        packed = to_e2m1<1>(packed, b[2] * inv, b[3] * inv);
        packed = to_e2m1<2>(packed, b[4] * inv, b[5] * inv);
        packed = to_e2m1<3>(packed, b[6] * inv, b[7] * inv);
        code[q] = fold_neg_zero(packed);
        if (ERR) {
            err = byte_err<0>(code[q], b, scale, err);
            err = byte_err<1>(code[q], b + 2, scale, err);
            err = byte_err<2>(code[q], b + 4, scale, err);
            err = byte_err<3>(code[q], b + 6, scale, err);
        }
    }
    return err;
}

// Block b's 32 fp32 values from the input (blocks are consecutive 32-element
// runs of the row-major [rows, K] input):
//   kInNvfp4  16 bytes of e2m1 codes (even k in the low nibble) and two e4m3
//             scales: w = e2m1 * (e4m3 / divisor), the division first (IEEE)
//   kInBf16   64 bytes of bf16: w = the value, widened exactly
//   kInFp8Ch  32 bytes of e4m3 and the row's fp32 scale: w = e4m3 * scale
constexpr int kInNvfp4 = 0, kInBf16 = 1, kInFp8Ch = 2;

// Partitions of one launch: consecutive block ranges, each with its divisor
// (NVFP4) and its first workgroup; the other inputs take one partition.
constexpr int kMaxParts = 16;
constexpr int kIters = 8;                                  // blocks per lane and workgroup
constexpr int64_t kWgBlocks = (int64_t)kThreads * kIters;
struct QuantIn {
    const uint8_t* data;        // codes or values of the rows
    const void* aux;            // nvfp4: e4m3 scale pairs; fp8: fp32 row scales
    int64_t blocks_per_row;     // fp8: the row of a block
    int n_parts;
    int64_t part_begin[kMaxParts + 1];   // first block of each partition; [n_parts] = the end
    int64_t wg_begin[kMaxParts + 1];     // first workgroup of each partition; [n_parts] = the grid
    float divisor[kMaxParts];            // nvfp4 global divisor
};

// Exact decodes through the matrix-format conversion instructions (unit
// scale): the e2m1 values of the four bytes of a dword (code 8 gives -0, as
// unpack_e2m1 does) and the OCP e4m3 values of its four bytes.
template <int T>
__device__ __forceinline__ void e2m1_pair(uint32_t dw, float* out) {
    const auto g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(dw, 1.0f, T);
    out[0] = g[0];
    out[1] = g[1];
}
__device__ __forceinline__ void e2m1_x8(uint32_t dw, float* out) {
    e2m1_pair<0>(dw, out);
    e2m1_pair<1>(dw, out + 2);
    e2m1_pair<2>(dw, out + 4);
    e2m1_pair<3>(dw, out + 6);
}
__device__ __forceinline__ void e4m3_x4(uint32_t dw, float* out) {
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(dw, 1.0f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(dw, 1.0f, true);
    out[0] = lo[0];
    out[1] = lo[1];
    out[2] = hi[0];
    out[3] = hi[1];
}

// Raw input of one block, loaded an iteration ahead of its encode
template <int IN> struct Raw;
template <> struct Raw<kInNvfp4> { uint4 c; uint32_t s; };
template <> struct Raw<kInBf16> { uint4 v[4]; };
template <> struct Raw<kInFp8Ch> { uint4 v[2]; float s; };

template <int IN>
__device__ __forceinline__ void load_raw(const QuantIn& in, int64_t b, Raw<IN>& r) {
    if constexpr (IN == kInNvfp4) {
        r.c = reinterpret_cast<const uint4*>(in.data)[b];
        r.s = reinterpret_cast<const uint16_t*>(in.aux)[b];
    } else if constexpr (IN == kInBf16) {
        const uint4* p = reinterpret_cast<const uint4*>(in.data) + 4 * b;
#pragma unroll
        for (int q = 0; q < 4; ++q) r.v[q] = p[q];
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(in.data) + 2 * b;
        r.v[0] = p[0];
        r.v[1] = p[1];
        // the row of block b (32-bit division: the entry point keeps the block
        // count below 2^32)
        r.s = reinterpret_cast<const float*>(in.aux)[(uint32_t)b / (uint32_t)in.blocks_per_row];
    }
}

template <int IN>
__device__ __forceinline__ void decode_block(const Raw<IN>& r, float divisor, float (&w)[32]) {
    if constexpr (IN == kInNvfp4) {
        float sv[4];
        e4m3_x4(r.s, sv);
        const float s0 = sv[0] / divisor;  // IEEE division
        const float s1 = sv[1] / divisor;
        const uint32_t dw[4] = {r.c.x, r.c.y, r.c.z, r.c.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) e2m1_x8(dw[q], w + 8 * q);
#pragma unroll
        for (int j = 0; j < 32; ++j) w[j] = w[j] * (j < 16 ? s0 : s1);
    } else if constexpr (IN == kInBf16) {
        uint32_t dw[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            dw[4 * q] = r.v[q].x; dw[4 * q + 1] = r.v[q].y; dw[4 * q + 2] = r.v[q].z; dw[4 * q + 3] = r.v[q].w;
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) w[j] = bf16_to_f32((dw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
    } else {
        const uint32_t dw[8] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w, r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w};
#pragma unroll
        for (int q = 0; q < 8; ++q) e4m3_x4(dw[q], w + 4 * q);
#pragma unroll
        for (int j = 0; j < 32; ++j) w[j] = w[j] * r.s;
    }
}

// One block: the exponent by the rule (returned) and the codes; the chosen
// error and the sum of squares go into the lane's statistics.
template <int IN, int MODE, bool STATS>
__device__ __forceinline__ int requant_encode(const Raw<IN>& r, float divisor, uint32_t (&code)[4],
                                              double& err_sum, double& ssq_sum) {
    float w[32];
    decode_block<IN>(r, divisor, w);
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(w[j]));
    int e;
    float err;
    if (MODE == W4A8_EXP_MSE) {
        const int e0 = block_exponent(amax, W4A8_EXP_NOCLIP);
        err = encode_block<true>(w, e0, code);
        e = e0;
        if (e0 - 1 >= -127) {
            uint32_t code1[4];
            const float r1 = encode_block<true>(w, e0 - 1, code1);
            if (r1 < err) {
                err = r1;
                e = e0 - 1;
#pragma unroll
                for (int q = 0; q < 4; ++q) code[q] = code1[q];
            }
        }
    } else {
        e = block_exponent(amax, MODE);
        err = encode_block<STATS>(w, e, code);
    }
    if (STATS) {
        err_sum += (double)err;
#pragma unroll
        for (int j = 0; j < 32; ++j) ssq_sum += (double)w[j] * (double)w[j];
    }
    return e;
}

// ... stored at block b of the row-major outputs
template <int IN, int MODE, bool STATS>
__device__ __forceinline__ void requant_block(const Raw<IN>& r, float divisor, int64_t b,
                                              uint4* __restrict__ out_packed, uint8_t* __restrict__ out_e8m0,
                                              double& err_sum, double& ssq_sum) {
    uint32_t code[4];
    const int e = requant_encode<IN, MODE, STATS>(r, divisor, code, err_sum, ssq_sum);
    out_packed[b] = make_uint4(code[0], code[1], code[2], code[3]);
    out_e8m0[b] = (uint8_t)(e + 127);
}

template <int IN, int MODE, bool STATS>
__global__ __launch_bounds__(kThreads) void requant_kernel(QuantIn in, uint4* __restrict__ out_packed,
                                                           uint8_t* __restrict__ out_e8m0,
                                                           double* __restrict__ stats) {
    // this workgroup's partition and block range (uniform: a scan over the
    // launch's table with constant indices)
    const int64_t wg = blockIdx.x;
    int p = 0;
#pragma unroll
    for (int i = 1; i < kMaxParts; ++i)
        if (i < in.n_parts && wg >= in.wg_begin[i]) p = i;
    int64_t lo = 0, hi = 0;
    float divisor = 1.0f;
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i)
        if (i == p) {
            lo = in.part_begin[i] + (wg - in.wg_begin[i]) * kWgBlocks;
            hi = min(lo + kWgBlocks, in.part_begin[i + 1]);
            divisor = in.divisor[i];
        }
    double err_sum = 0.0, ssq_sum = 0.0;
    // iteration it encodes block lo + it * kThreads + tid; a lane past the
    // range's end loads its last block and stores nothing
    auto blk = [&](int it) { return lo + (int64_t)it * kThreads + threadIdx.x; };
    Raw<IN> r0, r1;
    load_raw<IN>(in, min(blk(0), hi - 1), r0);
#pragma unroll
    for (int it = 0; it < kIters; it += 2) {
        load_raw<IN>(in, min(blk(it + 1), hi - 1), r1);
        if (blk(it) < hi)
            requant_block<IN, MODE, STATS>(r0, divisor, blk(it), out_packed, out_e8m0, err_sum, ssq_sum);
        if (it + 2 < kIters) load_raw<IN>(in, min(blk(it + 2), hi - 1), r0);
        if (blk(it + 1) < hi)
            requant_block<IN, MODE, STATS>(r1, divisor, blk(it + 1), out_packed, out_e8m0, err_sum, ssq_sum);
    }
    if (STATS) {
        // wavefront then workgroup reduction, one pair of atomics per workgroup
        // into its partition's slots
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            err_sum += __shfl_xor(err_sum, off);
            ssq_sum += __shfl_xor(ssq_sum, off);
        }
        __shared__ double red[2][kThreads / 64];
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        if (lane == 0) {
            red[0][wave] = err_sum;
            red[1][wave] = ssq_sum;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            double a = 0.0, s = 0.0;
            for (int i = 0; i < kThreads / 64; ++i) {
                a += red[0][i];
                s += red[1][i];
            }
            atomicAdd(&stats[2 * p], a);
            atomicAdd(&stats[2 * p + 1], s);
        }
    }
}
static_assert(kIters % 2 == 0, "the loop above takes iterations in pairs");

// The same encoder writing the matrix-core fragment order of the GEMM's
// prepared weights directly (the layout the load-time repack writes from the
// row-major arrays): one wave per 16-row tile t and 4-step chunk c, lane
// L = n + 16 g on row 16 t + n and K-blocks 4 s + g of the chunk's steps s.
// Each step's 16 code bytes go to lane L's slot of the tile's 1 KiB block for
// that step, the four e8m0 bytes to lane L's dword of the chunk's 256-byte
// record (byte u: step 4 c + u), so a wave stores whole 1 KiB and 256-byte
// runs.  Rows past the weight and steps past K are padding: code 0 and e8m0
// 127 (the repack's).  The partition (divisor) is the row's; no statistics.
template <int IN, int MODE>
__global__ __launch_bounds__(kThreads) void requant_frag_kernel(QuantIn in, int64_t rows, int64_t K, int64_t tiles,
                                                                int c_pad, uint4* __restrict__ wt,
                                                                uint32_t* __restrict__ st) {
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (unit >= tiles * c_pad) return;
    const int64_t t = unit / c_pad;
    const int c = (int)(unit - t * c_pad);
    const int64_t row = 16 * t + (lane & 15);
    const int g = lane >> 4, steps = (int)(K / 128);
    const int64_t bpr = K / 32;
    float divisor = 1.0f;
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i)
        if (i < in.n_parts && row * bpr >= in.part_begin[i]) divisor = in.divisor[i];
    // the chunk's four blocks loaded before any is encoded (block 0 for padding)
    Raw<IN> r[4];
    bool real[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int s = 4 * c + j;
        real[j] = row < rows && s < steps;
        load_raw<IN>(in, real[j] ? row * bpr + 4 * s + g : 0, r[j]);
    }
    double none = 0.0;
    uint32_t e8 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t code[4] = {0u, 0u, 0u, 0u};
        uint32_t byte = 127u;
        if (real[j]) byte = (uint32_t)(requant_encode<IN, MODE, false>(r[j], divisor, code, none, none) + 127);
        wt[(t * 4 * c_pad + 4 * c + j) * 64 + lane] = make_uint4(code[0], code[1], code[2], code[3]);
        e8 |= byte << (8 * j);
    }
    st[(t * c_pad + c) * 64 + lane] = e8;
}

__global__ void fill_zero_f64(double* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0;
}
__global__ void fill_zero_u32(uint32_t* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

template <int IN, int MODE>
hipError_t launch_mode(const QuantIn& in, uint8_t* mx_packed, uint8_t* mx_e8m0, double* stats,
                       hipStream_t stream) {
    const int64_t grid = in.wg_begin[in.n_parts];
    if (grid <= 0) return hipSuccess;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    if (stats)
        hipLaunchKernelGGL((requant_kernel<IN, MODE, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, in,
                           (uint4*)mx_packed, mx_e8m0, stats);
    else
        hipLaunchKernelGGL((requant_kernel<IN, MODE, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           in, (uint4*)mx_packed, mx_e8m0, stats);
    return hipGetLastError();
}

template <int IN>
hipError_t launch_in(const QuantIn& in, int mode, uint8_t* mx_packed, uint8_t* mx_e8m0, double* stats,
                     hipStream_t stream) {
    switch (mode) {
        case W4A8_EXP_OCP:
            return launch_mode<IN, W4A8_EXP_OCP>(in, mx_packed, mx_e8m0, stats, stream);
        case W4A8_EXP_NOCLIP:
            return launch_mode<IN, W4A8_EXP_NOCLIP>(in, mx_packed, mx_e8m0, stats, stream);
        default:
            return launch_mode<IN, W4A8_EXP_MSE>(in, mx_packed, mx_e8m0, stats, stream);
    }
}

template <int IN>
hipError_t launch_frag(const QuantIn& in, int mode, int64_t rows, int64_t K, uint8_t* wt, uint8_t* st,
                       hipStream_t stream) {
    const int64_t tiles = (rows + 15) / 16, c_pad = (K / 128 + 3) / 4;
    const int64_t grid = (tiles * c_pad + kThreads / 64 - 1) / (kThreads / 64);
    if (grid <= 0) return hipSuccess;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    uint4* w = reinterpret_cast<uint4*>(wt);
    uint32_t* s = reinterpret_cast<uint32_t*>(st);
    const dim3 g((unsigned)grid), b(kThreads);
    if (mode == W4A8_EXP_OCP)
        hipLaunchKernelGGL((requant_frag_kernel<IN, W4A8_EXP_OCP>), g, b, 0, stream, in, rows, K, tiles, (int)c_pad, w, s);
    else if (mode == W4A8_EXP_NOCLIP)
        hipLaunchKernelGGL((requant_frag_kernel<IN, W4A8_EXP_NOCLIP>), g, b, 0, stream, in, rows, K, tiles, (int)c_pad, w,
                           s);
    else
        hipLaunchKernelGGL((requant_frag_kernel<IN, W4A8_EXP_MSE>), g, b, 0, stream, in, rows, K, tiles, (int)c_pad, w, s);
    return hipGetLastError();
}

// the launch table of partitions 0..n-1 with cnt[i] blocks each
void plan_parts(QuantIn& in, const int64_t* cnt, const float* divisor, int n) {
    in.n_parts = n;
    in.part_begin[0] = 0;
    in.wg_begin[0] = 0;
    for (int i = 0; i < n; ++i) {
        in.part_begin[i + 1] = in.part_begin[i] + cnt[i];
        in.wg_begin[i + 1] = in.wg_begin[i] + (cnt[i] + kWgBlocks - 1) / kWgBlocks;
        in.divisor[i] = divisor ? divisor[i] : 1.0f;
    }
}

}  // namespace

int requant_max_parts() { return kMaxParts; }

hipError_t launch_requant(const uint8_t* nv_packed, const uint8_t* nv_scale, const int64_t* part_blocks,
                          const float* part_divisor, int n_parts, int mode, uint8_t* mx_packed,
                          uint8_t* mx_e8m0, double* stats, hipStream_t stream) {
    if (n_parts < 1 || n_parts > kMaxParts) return hipErrorInvalidValue;
    QuantIn in{};
    in.data = nv_packed;
    in.aux = nv_scale;
    in.blocks_per_row = 1;
    plan_parts(in, part_blocks, part_divisor, n_parts);
    return launch_in<kInNvfp4>(in, mode, mx_packed, mx_e8m0, stats, stream);
}

hipError_t launch_quant_bf16(const uint16_t* w, int64_t rows, int64_t K, int mode, uint8_t* mx_packed,
                             uint8_t* mx_e8m0, double* stats, hipStream_t stream) {
    QuantIn in{};
    in.data = reinterpret_cast<const uint8_t*>(w);
    in.blocks_per_row = K / 32;
    const int64_t n = rows * (K / 32);
    plan_parts(in, &n, nullptr, 1);
    return launch_in<kInBf16>(in, mode, mx_packed, mx_e8m0, stats, stream);
}

hipError_t launch_quant_fp8ch(const uint8_t* w, const float* row_scale, int64_t rows, int64_t K, int mode,
                              uint8_t* mx_packed, uint8_t* mx_e8m0, double* stats, hipStream_t stream) {
    QuantIn in{};
    in.data = w;
    in.aux = row_scale;
    in.blocks_per_row = K / 32;
    const int64_t n = rows * (K / 32);
    plan_parts(in, &n, nullptr, 1);
    return launch_in<kInFp8Ch>(in, mode, mx_packed, mx_e8m0, stats, stream);
}

// the three load-time encoders writing fragment order (K % 128 == 0; at most
// requant_max_parts() partitions in one launch)
hipError_t launch_requant_prepared(const uint8_t* nv_packed, const uint8_t* nv_scale, const int64_t* part_blocks,
                                   const float* part_divisor, int n_parts, int64_t rows, int64_t K, int mode,
                                   uint8_t* wt, uint8_t* st, hipStream_t stream) {
    if (n_parts < 1 || n_parts > kMaxParts || K % 128 != 0) return hipErrorInvalidValue;
    QuantIn in{};
    in.data = nv_packed;
    in.aux = nv_scale;
    in.blocks_per_row = 1;
    plan_parts(in, part_blocks, part_divisor, n_parts);
    return launch_frag<kInNvfp4>(in, mode, rows, K, wt, st, stream);
}

hipError_t launch_quant_bf16_prepared(const uint16_t* w, int64_t rows, int64_t K, int mode, uint8_t* wt,
                                      uint8_t* st, hipStream_t stream) {
    if (K % 128 != 0) return hipErrorInvalidValue;
    QuantIn in{};
    in.data = reinterpret_cast<const uint8_t*>(w);
    in.blocks_per_row = K / 32;
    const int64_t n = rows * (K / 32);
    plan_parts(in, &n, nullptr, 1);
    return launch_frag<kInBf16>(in, mode, rows, K, wt, st, stream);
}

hipError_t launch_quant_fp8ch_prepared(const uint8_t* w, const float* row_scale, int64_t rows, int64_t K, int mode,
                                       uint8_t* wt, uint8_t* st, hipStream_t stream) {
    if (K % 128 != 0) return hipErrorInvalidValue;
    QuantIn in{};
    in.data = w;
    in.aux = row_scale;
    in.blocks_per_row = K / 32;
    const int64_t n = rows * (K / 32);
    plan_parts(in, &n, nullptr, 1);
    return launch_frag<kInFp8Ch>(in, mode, rows, K, wt, st, stream);
}

hipError_t launch_fill_zero_f64(double* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_f64, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_fill_zero_u32(uint32_t* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

}  // namespace w4a8
