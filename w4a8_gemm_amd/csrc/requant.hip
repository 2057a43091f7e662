// requant.hip -- NVFP4 -> MXFP4 requantization on gfx950.
//
// "radiance_nvfp4.py": dequant_nvfp4 (W = e2m1 * e4m3 scale / global divisor),
// _block_exponent (ocp / noclip rules), e2m1_index (nearest grid point, ties to
// the even index, saturating at 6), _encode_blocks (squared error per block),
// quant_mxfp4 (mse picks noclip or noclip-1; sign bit only on nonzero codes;
// e8m0 = e + 127).
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
// element order; writes 4-bit magnitude indices (no sign) into idx.
__device__ __forceinline__ float encode_block(const float* w, int e, uint32_t* idx) {
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, normal for e in [-127, 126]
    const float scale = ldexpf(1.0f, e);                            // 2^e, exact (subnormal at -127)
    float err = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) idx[q] = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float v = w[j] * inv;  // == w / 2^e, both correctly rounded
        const float a = fabsf(v);
        const uint32_t i = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                           (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                           (uint32_t)(a > 5.0f);
        const float sgn = v > 0.0f ? 1.0f : (v < 0.0f ? -1.0f : 0.0f);
        const float q = e2m1_mag(i) * sgn * scale;
        const float d = q - w[j];
        const float sq = d * d;
        err = err + sq;
        idx[j >> 3] |= i << (4 * (j & 7));
    }
    return err;
}

template <int MODE, bool STATS>
__global__ __launch_bounds__(kThreads) void requant_kernel(
    const uint4* __restrict__ in_packed, const uint16_t* __restrict__ in_scale, float divisor,
    int64_t nblocks, uint4* __restrict__ out_packed, uint8_t* __restrict__ out_e8m0,
    double* __restrict__ stats) {
    double err_sum = 0.0, ssq_sum = 0.0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += stride) {
        const uint4 p = in_packed[b];
        const uint32_t sc = in_scale[b];
        const float s0 = e4m3_to_f32(sc & 0xFFu) / divisor;  // IEEE division
        const float s1 = e4m3_to_f32(sc >> 8) / divisor;
        const uint32_t dw[4] = {p.x, p.y, p.z, p.w};
        float w[32];
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const uint32_t c = (dw[j >> 3] >> (4 * (j & 7))) & 15u;
            const float val = (c & 8u) ? -e2m1_mag(c & 7u) : e2m1_mag(c & 7u);
            w[j] = val * (j < 16 ? s0 : s1);
            amax = fmaxf(amax, fabsf(w[j]));
        }
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

template <int MODE>
hipError_t launch_mode(const uint8_t* nv_packed, const uint8_t* nv_scale, float divisor,
                       int64_t nblocks, uint8_t* mx_packed, uint8_t* mx_e8m0, double* stats,
                       hipStream_t stream) {
    // enough workgroups to fill 256 CUs several times over; lanes loop beyond that
    const int64_t want = (nblocks + kThreads - 1) / kThreads;
    const int grid = (int)(want < 4096 ? want : 4096);
    if (stats)
        hipLaunchKernelGGL((requant_kernel<MODE, true>), dim3(grid), dim3(kThreads), 0, stream,
                           (const uint4*)nv_packed, (const uint16_t*)nv_scale, divisor, nblocks,
                           (uint4*)mx_packed, mx_e8m0, stats);
    else
        hipLaunchKernelGGL((requant_kernel<MODE, false>), dim3(grid), dim3(kThreads), 0, stream,
                           (const uint4*)nv_packed, (const uint16_t*)nv_scale, divisor, nblocks,
                           (uint4*)mx_packed, mx_e8m0, stats);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_requant(const uint8_t* nv_packed, const uint8_t* nv_scale, float divisor,
                          int64_t nblocks, int mode, uint8_t* mx_packed, uint8_t* mx_e8m0,
                          double* stats, hipStream_t stream) {
    if (nblocks <= 0) return hipSuccess;
    switch (mode) {
        case W4A8_EXP_OCP:
            return launch_mode<W4A8_EXP_OCP>(nv_packed, nv_scale, divisor, nblocks, mx_packed,
                                             mx_e8m0, stats, stream);
        case W4A8_EXP_NOCLIP:
            return launch_mode<W4A8_EXP_NOCLIP>(nv_packed, nv_scale, divisor, nblocks, mx_packed,
                                                mx_e8m0, stats, stream);
        default:
            return launch_mode<W4A8_EXP_MSE>(nv_packed, nv_scale, divisor, nblocks, mx_packed,
                                             mx_e8m0, stats, stream);
    }
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
