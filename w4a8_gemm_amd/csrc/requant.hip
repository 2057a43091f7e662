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
// wavefront reads and writes contiguous 1 KiB / 128 B / 1 KiB / 64 B runs.  The
// pass is bandwidth/ALU bound; no LDS is needed.  Squared errors are summed in
// fp32 in element order 0..31, each square rounded first, with no fused
// multiply-add (the file is compiled with -ffp-contract=off), so the mse
// decision is a fixed function of the inputs.
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

// Encode one block at exponent e.  Returns the fp32 squared error summed in
// element order; writes 4-bit magnitude indices (no sign) into idx.  The index
// of |w| / 2^e comes from the matrix-format conversion instructions, whose
// rounding is the page's e2m1_index on magnitudes (nearest grid point, ties
// to the even index -- the index's low bit is the mantissa bit -- and values
// above 6 saturating at 6; checked against the rule for every magnitude class
// on gfx950); the grid value comes back through the reverse conversion.
template <int T>
__device__ __forceinline__ uint32_t to_e2m1(uint32_t old, float a0, float a1) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a0, a1, 1.0f, T);   // byte T <- indices of a0, a1
}
// squared errors of the two elements of byte T (grid values scaled by 2^e,
// signed like w), added to err in element order
template <int T>
__device__ __forceinline__ float byte_err(uint32_t packed, const float* w2, float scale, float err) {
    const auto g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, T);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float qv = copysignf(g[u] * scale, w2[u]);   // exact
        const float d = qv - w2[u];
        const float sq = d * d;
        err = err + sq;
    }
    return err;
}

__device__ __forceinline__ float encode_block(const float* w, int e, uint32_t* idx) {
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, normal for e in [-127, 126]
    const float scale = ldexpf(1.0f, e);                            // 2^e, exact (subnormal at -127)
    float err = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float* b = w + 8 * q;
        // |w / 2^e|, each product correctly rounded
        uint32_t packed = to_e2m1<0>(0u, fabsf(b[0] * inv), fabsf(b[1] * inv));
        packed = to_e2m1<1>(packed, fabsf(b[2] * inv), fabsf(b[3] * inv));
        packed = to_e2m1<2>(packed, fabsf(b[4] * inv), fabsf(b[5] * inv));
        packed = to_e2m1<3>(packed, fabsf(b[6] * inv), fabsf(b[7] * inv));
        idx[q] = packed;
        err = byte_err<0>(packed, b, scale, err);
        err = byte_err<1>(packed, b + 2, scale, err);
        err = byte_err<2>(packed, b + 4, scale, err);
        err = byte_err<3>(packed, b + 6, scale, err);
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

struct QuantIn {
    const uint8_t* data;        // codes or values of the rows
    const void* aux;            // nvfp4: e4m3 scale pairs; fp8: fp32 row scales
    float divisor;              // nvfp4 global divisor
    int64_t blocks_per_row;     // fp8: the row of a block
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

template <int IN>
__device__ __forceinline__ void load_block(const QuantIn& in, int64_t b, float (&w)[32]) {
    if constexpr (IN == kInNvfp4) {
        const uint4 p = reinterpret_cast<const uint4*>(in.data)[b];
        const uint32_t sc = reinterpret_cast<const uint16_t*>(in.aux)[b];
        float sv[4];
        e4m3_x4(sc, sv);
        const float s0 = sv[0] / in.divisor;  // IEEE division
        const float s1 = sv[1] / in.divisor;
        const uint32_t dw[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) e2m1_x8(dw[q], w + 8 * q);
#pragma unroll
        for (int j = 0; j < 32; ++j) w[j] = w[j] * (j < 16 ? s0 : s1);
    } else if constexpr (IN == kInBf16) {
        const uint4* p = reinterpret_cast<const uint4*>(in.data) + 4 * b;
        uint32_t dw[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = p[q];
            dw[4 * q] = v.x; dw[4 * q + 1] = v.y; dw[4 * q + 2] = v.z; dw[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) w[j] = bf16_to_f32((dw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(in.data) + 2 * b;
        // the row of block b (32-bit division: the entry point keeps the block
        // count below 2^32)
        const float s = reinterpret_cast<const float*>(in.aux)[(uint32_t)b / (uint32_t)in.blocks_per_row];
        const uint4 v0 = p[0], v1 = p[1];
        const uint32_t dw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) e4m3_x4(dw[q], w + 4 * q);
#pragma unroll
        for (int j = 0; j < 32; ++j) w[j] = w[j] * s;
    }
}

template <int IN, int MODE, bool STATS>
__global__ __launch_bounds__(kThreads) void requant_kernel(
    QuantIn in, int64_t nblocks, uint4* __restrict__ out_packed, uint8_t* __restrict__ out_e8m0,
    double* __restrict__ stats) {
    double err_sum = 0.0, ssq_sum = 0.0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += stride) {
        float w[32];
        load_block<IN>(in, b, w);
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(w[j]));
        uint32_t idx[4];
        int e;
        float err;
        if (MODE == W4A8_EXP_MSE) {
            const int e0 = block_exponent(amax, W4A8_EXP_NOCLIP);
            err = encode_block(w, e0, idx);
            e = e0;
            if (e0 - 1 >= -127) {
                uint32_t idx1[4];
                const float r1 = encode_block(w, e0 - 1, idx1);
                if (r1 < err) {
                    err = r1;
                    e = e0 - 1;
#pragma unroll
                    for (int q = 0; q < 4; ++q) idx[q] = idx1[q];
                }
            }
        } else {
            e = block_exponent(amax, MODE);
            err = encode_block(w, e, idx);
        }
        // sign bit only where the index is nonzero (a negative zero keeps code 0)
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t sgn = 0u;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int j = 8 * q + t;
                const uint32_t nz = (idx[q] >> (4 * t)) & 7u;
                if (nz && (__float_as_uint(w[j]) >> 31)) sgn |= 8u << (4 * t);
            }
            o[q] = idx[q] | sgn;
        }
        out_packed[b] = make_uint4(o[0], o[1], o[2], o[3]);
        out_e8m0[b] = (uint8_t)(e + 127);
        if (STATS) {
            err_sum += (double)err;
#pragma unroll
            for (int j = 0; j < 32; ++j) ssq_sum += (double)w[j] * (double)w[j];
        }
    }
    if (STATS) {
        // wavefront then workgroup reduction, one pair of atomics per workgroup
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
            atomicAdd(&stats[0], a);
            atomicAdd(&stats[1], s);
        }
    }
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
hipError_t launch_mode(const QuantIn& in, int64_t nblocks, uint8_t* mx_packed, uint8_t* mx_e8m0,
                       double* stats, hipStream_t stream) {
    // enough workgroups to fill 256 CUs several times over; lanes loop beyond that
    const int64_t want = (nblocks + kThreads - 1) / kThreads;
    const int grid = (int)(want < 4096 ? want : 4096);
    if (stats)
        hipLaunchKernelGGL((requant_kernel<IN, MODE, true>), dim3(grid), dim3(kThreads), 0, stream, in, nblocks,
                           (uint4*)mx_packed, mx_e8m0, stats);
    else
        hipLaunchKernelGGL((requant_kernel<IN, MODE, false>), dim3(grid), dim3(kThreads), 0, stream, in,
                           nblocks, (uint4*)mx_packed, mx_e8m0, stats);
    return hipGetLastError();
}

template <int IN>
hipError_t launch_in(const QuantIn& in, int64_t nblocks, int mode, uint8_t* mx_packed, uint8_t* mx_e8m0,
                     double* stats, hipStream_t stream) {
    if (nblocks <= 0) return hipSuccess;
    switch (mode) {
        case W4A8_EXP_OCP:
            return launch_mode<IN, W4A8_EXP_OCP>(in, nblocks, mx_packed, mx_e8m0, stats, stream);
        case W4A8_EXP_NOCLIP:
            return launch_mode<IN, W4A8_EXP_NOCLIP>(in, nblocks, mx_packed, mx_e8m0, stats, stream);
        default:
            return launch_mode<IN, W4A8_EXP_MSE>(in, nblocks, mx_packed, mx_e8m0, stats, stream);
    }
}

}  // namespace

hipError_t launch_requant(const uint8_t* nv_packed, const uint8_t* nv_scale, float divisor,
                          int64_t nblocks, int mode, uint8_t* mx_packed, uint8_t* mx_e8m0,
                          double* stats, hipStream_t stream) {
    const QuantIn in{nv_packed, nv_scale, divisor, 1};
    return launch_in<kInNvfp4>(in, nblocks, mode, mx_packed, mx_e8m0, stats, stream);
}

hipError_t launch_quant_bf16(const uint16_t* w, int64_t rows, int64_t K, int mode, uint8_t* mx_packed,
                             uint8_t* mx_e8m0, double* stats, hipStream_t stream) {
    const QuantIn in{reinterpret_cast<const uint8_t*>(w), nullptr, 1.0f, K / 32};
    return launch_in<kInBf16>(in, rows * (K / 32), mode, mx_packed, mx_e8m0, stats, stream);
}

hipError_t launch_quant_fp8ch(const uint8_t* w, const float* row_scale, int64_t rows, int64_t K, int mode,
                              uint8_t* mx_packed, uint8_t* mx_e8m0, double* stats, hipStream_t stream) {
    const QuantIn in{w, row_scale, 1.0f, K / 32};
    return launch_in<kInFp8Ch>(in, rows * (K / 32), mode, mx_packed, mx_e8m0, stats, stream);
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
