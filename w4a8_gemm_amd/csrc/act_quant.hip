// act_quant.hip -- dynamic per-token fp8 (E4M3FN) activation quantization.
//
// "radiance_autoround.py", autoround_linear: activations become e4m3 codes with
// one fp32 scale per token (row) before the W4A8 GEMM.  The pages leave the
// arithmetic to a library op; the plain reading used here:
//   s = amax_k |x[m,k]| / 448   (1 for an all-zero row)
//   code = e4m3 round-to-nearest-even of x / s, saturating at 448, sign kept.
// Rows of up to 256 * 8 * 16 elements (and 16-byte aligned) are split over
// ceil(K / 8 / 256) workgroups when the rows are fewer than the CUs (else one
// workgroup per row): each reads the whole row once into registers
// -- every load issued before the first use, so the row costs one memory
// latency -- takes the block max (wavefront butterfly, then LDS across the
// four waves) and divides and encodes its share of the row from registers.
// Longer or unaligned rows take a two-pass form, one workgroup per row, that
// re-reads the row from L2.
#include "w4a8_internal.h"

#pragma clang fp contract(off)

namespace w4a8 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    __shared__ float red[kThreads / 64];
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
    return r;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void act_quant_kernel(const uint16_t* __restrict__ x,
                                                             int64_t K, int64_t ldx,
                                                             uint8_t* __restrict__ x8,
                                                             float* __restrict__ xs) {
    const int64_t m = blockIdx.x;
    const uint16_t* row = x + m * ldx;
    uint8_t* orow = x8 + m * K;
    float amax = 0.0f;
    if (VEC) {
        const uint4* r4 = reinterpret_cast<const uint4*>(row);
        for (int64_t c = threadIdx.x; c < K / 8; c += kThreads) {
            const uint4 v = r4[c];
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                amax = fmaxf(amax, fabsf(bf16_to_f32(d[q] & 0xFFFFu)));
                amax = fmaxf(amax, fabsf(bf16_to_f32(d[q] >> 16)));
            }
        }
    } else {
        for (int64_t k = threadIdx.x; k < K; k += kThreads)
            amax = fmaxf(amax, fabsf(bf16_to_f32(row[k])));
    }
    amax = block_max(amax);
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;  // IEEE division
    if (threadIdx.x == 0) xs[m] = s;
    if (VEC) {
        const uint4* r4 = reinterpret_cast<const uint4*>(row);
        uint2* o2 = reinterpret_cast<uint2*>(orow);
        for (int64_t c = threadIdx.x; c < K / 8; c += kThreads) {
            const uint4 v = r4[c];
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
            uint32_t o[2] = {0u, 0u};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = f32_to_e4m3_rne_sat(bf16_to_f32(d[q] & 0xFFFFu) / s);
                const uint32_t hi = f32_to_e4m3_rne_sat(bf16_to_f32(d[q] >> 16) / s);
                o[q >> 1] |= (lo | (hi << 8)) << (16 * (q & 1));
            }
            o2[c] = make_uint2(o[0], o[1]);
        }
    } else {
        for (int64_t k = threadIdx.x; k < K; k += kThreads)
            orow[k] = (uint8_t)f32_to_e4m3_rne_sat(bf16_to_f32(row[k]) / s);
    }
}

// Rows split over S workgroups (S = ceil(items / threads), so that a thread
// encodes at most one 8-value item): every workgroup of a row reads the whole
// row for its amax (all loads issued before the first use), then encodes only
// its share of the items, [n8 c / S, n8 (c + 1) / S); the row's first
// workgroup writes the scale.  The divide-and-encode of a row, about 25
// vector instructions per value, is then spread over S CUs instead of one.
template <int R>
__global__ __launch_bounds__(kThreads) void act_quant_split_kernel(const uint16_t* __restrict__ x, int64_t K,
                                                                   int64_t ldx, uint8_t* __restrict__ x8,
                                                                   float* __restrict__ xs,
                                                                   uint8_t* __restrict__ x8s, int S, int M) {
    const int64_t m = blockIdx.x / S;
    const int c = (int)(blockIdx.x - m * S);
    const uint4* r4 = reinterpret_cast<const uint4*>(x + m * ldx);
    const int n8 = (int)(K / 8);
    uint4 v[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int it = threadIdx.x + kThreads * i;
        v[i] = it < n8 ? r4[it] : make_uint4(0, 0, 0, 0);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const uint32_t d[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            amax = fmaxf(amax, fabsf(bf16_to_f32(d[q] & 0xFFFFu)));
            amax = fmaxf(amax, fabsf(bf16_to_f32(d[q] >> 16)));
        }
    }
    amax = block_max(amax);
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;  // IEEE division
    if (c == 0 && threadIdx.x == 0) xs[m] = s;
    const int lo = (int)((int64_t)n8 * c / S), hi = (int)((int64_t)n8 * (c + 1) / S);
    uint2* o2 = reinterpret_cast<uint2*>(x8 + m * K);
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int it = threadIdx.x + kThreads * i;
        if (it < lo || it >= hi) continue;
        const uint32_t d[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t l = f32_to_e4m3_rne_sat(bf16_to_f32(d[q] & 0xFFFFu) / s);
            const uint32_t h = f32_to_e4m3_rne_sat(bf16_to_f32(d[q] >> 16) / s);
            o[q >> 1] |= (l | (h << 8)) << (16 * (q & 1));
        }
        o2[it] = make_uint2(o[0], o[1]);
        if (x8s)
            *reinterpret_cast<uint2*>(x8s + (int64_t)(it >> 4) * 128 * M + 128 * m + 8 * (it & 15)) =
                make_uint2(o[0], o[1]);
    }
}

// fewer rows than CUs: each split over S workgroups; more: one workgroup per
// row (each workgroup re-reads its whole row, so a split would multiply the
// HBM reads of a prefill-sized launch)
template <int R>
hipError_t launch_split(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* x8, float* xs, uint8_t* x8s,
                        hipStream_t stream) {
    const int S = M < 256 ? (int)((K / 8 + kThreads - 1) / kThreads) : 1;
    if (M * S > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(act_quant_split_kernel<R>, dim3((unsigned)(M * S)), dim3(kThreads), 0, stream, x, K, ldx, x8,
                       xs, x8s, S, (int)M);
    return hipGetLastError();
}

// the single-pass rows
hipError_t launch_rows(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* x8, float* xs, uint8_t* x8s,
                       hipStream_t stream) {
    const int64_t per_thread = (K / 8 + kThreads - 1) / kThreads;   // uint4 per thread
    if (per_thread <= 1) return launch_split<1>(x, M, K, ldx, x8, xs, x8s, stream);
    if (per_thread <= 2) return launch_split<2>(x, M, K, ldx, x8, xs, x8s, stream);
    if (per_thread <= 4) return launch_split<4>(x, M, K, ldx, x8, xs, x8s, stream);
    if (per_thread <= 8) return launch_split<8>(x, M, K, ldx, x8, xs, x8s, stream);
    return launch_split<16>(x, M, K, ldx, x8, xs, x8s, stream);
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* x8,
                            float* xs, hipStream_t stream) {
    const bool vec = (K % 8 == 0) && (ldx % 8 == 0) && ((uintptr_t)x % 16 == 0) &&
                     ((uintptr_t)x8 % 8 == 0);
    const int64_t per_thread = (K / 8 + kThreads - 1) / kThreads;   // uint4 per thread
    if (vec && per_thread <= 16) {
        return launch_rows(x, M, K, ldx, x8, xs, nullptr, stream);
    } else if (vec)
        hipLaunchKernelGGL(act_quant_kernel<true>, dim3((unsigned)M), dim3(kThreads), 0, stream, x,
                           K, ldx, x8, xs);
    else
        hipLaunchKernelGGL(act_quant_kernel<false>, dim3((unsigned)M), dim3(kThreads), 0, stream,
                           x, K, ldx, x8, xs);
    return hipGetLastError();
}

bool act_quant_sm_fits(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint8_t* x8) {
    return M >= 1 && K % 128 == 0 && ldx % 8 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)x8 % 8 == 0 &&
           (K / 8 + kThreads - 1) / kThreads <= 16;
}

hipError_t launch_act_quant_sm(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* x8, float* xs,
                               uint8_t* x8s, hipStream_t stream) {
    if (!act_quant_sm_fits(x, M, K, ldx, x8) || !x8s || (uintptr_t)x8s % 16 != 0) return hipErrorInvalidValue;
    return launch_rows(x, M, K, ldx, x8, xs, x8s, stream);
}

}  // namespace w4a8
