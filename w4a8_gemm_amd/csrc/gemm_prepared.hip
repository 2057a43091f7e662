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

// ---------------------------------------------------------------------------
// prepare: plain [N, K/2] codes + [N, K/32] e8m0 -> fragment order
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void prep_w_kernel(const uint8_t* __restrict__ wq, int N, int K,
                                                     int tiles, int s_pad, uint4* __restrict__ wt) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)tiles * s_pad * 64) return;
    const int L = (int)(i & 63);
    const int64_t blk = i >> 6;
    const int s = (int)(blk % s_pad), t = (int)(blk / s_pad);
    const int row = 16 * t + (L & 15), g = L >> 4;
    uint4 v = make_uint4(0, 0, 0, 0);
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

// ---------------------------------------------------------------------------
// decode band on prepared weights (M <= 32)
//
// Workgroup = 4 waves = 64 weight rows (one 16-row tile per wave) x one K split
// of whole 512-wide chunks.  The workgroup first copies the split's activations
// (all M rows) into LDS (rows padded by 16 bytes: the 16 column lanes of an
// MFMA fragment read then fall in distinct banks); each wave then streams its
// tile's weight blocks and scale dwords through a D-deep register ring, loads
// issued D-1 chunks ahead of the MFMAs (straight-line code between scheduling
// barriers, so each wait covers exactly the chunk about to be used; chunk
// indices past the end re-read the last chunk instead of branching).
// ---------------------------------------------------------------------------

struct PDecArgs {
    const uint8_t* x8;
    const float* xs;
    const uint4* wt;
    const uint32_t* st;
    uint16_t* out;
    float* partials;
    int M, N, K;
    int s_pad, c_pad;   // padded 128-steps and 4-step chunks per row tile
    int tiles;          // 16-row tiles (ceil(N / 16))
    int groups;         // workgroups per split (ceil(tiles / 4))
    int ks, c_per;      // K splits, chunks per split
};

template <int MT>
struct PChunk {
    uint4 w[4];
    uint32_t s;
};

__device__ __forceinline__ void pdec_load(const uint4* wp, const uint32_t* sp, int j, PChunk<1>& c) {
#pragma unroll
    for (int u = 0; u < 4; ++u) c.w[u] = wp[(4 * j + u) * 64];
    c.s = sp[j * 64];
}

template <int MT>
__device__ __forceinline__ void pdec_compute(const uint8_t* xl, int stride, int lane, int M, int j,
                                             const PChunk<1>& c, v4f (&acc)[MT]) {
    const int g = lane >> 4;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
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
    }
}

template <int MT, int D>
__global__ __launch_bounds__(256) void pdec_kernel(PDecArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t xl[];
    const int tg = blockIdx.x % a.groups, split = blockIdx.x / a.groups;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = tg * 4 + wave;
    const int c0 = split * a.c_per;
    const int c1 = min(a.c_pad, c0 + a.c_per);
    const int nch = c1 > c0 ? c1 - c0 : 0;
    const int kbase = c0 * 512, kr = nch * 512, stride = kr + 16;

    // activations of this split -> LDS (columns at or past K read as zero)
    const int per_row = kr / 16;
    for (int q = threadIdx.x; q < a.M * per_row; q += 256) {
        const int m = q / per_row, col = q - m * per_row;
        const int k = kbase + 16 * col;
        const uint4 v = k < a.K ? *reinterpret_cast<const uint4*>(a.x8 + (int64_t)m * a.K + k)
                                : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(xl + m * stride + 16 * col) = v;
    }
    __syncthreads();
    if (t >= a.tiles || nch == 0) return;   // no barrier follows

    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
    const uint4* wp = a.wt + ((int64_t)t * a.s_pad + 4 * (int64_t)c0) * 64 + lane;
    const uint32_t* sp = a.st + ((int64_t)t * a.c_pad + c0) * 64 + lane;

    PChunk<1> ring[D];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) pdec_load(wp, sp, min(d, nch - 1), ring[d]);
    for (int j = 0; j < nch; j += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            pdec_load(wp, sp, min(j + d + D - 1, nch - 1), ring[(d + D - 1) % D]);
            __builtin_amdgcn_sched_barrier(0);
            if (j + d < nch) pdec_compute<MT>(xl, stride, lane, a.M, j + d, ring[d], acc);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    const int g = lane >> 4;
    const int n0 = 16 * t + 4 * g;
    if (n0 >= a.N) return;
    const bool vec = (a.N & 3) == 0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + (lane & 15);
        if (m >= a.M) continue;
        if (a.ks == 1) {
            const float sm = a.xs[m];
            uint16_t* o = a.out + (int64_t)m * a.N + n0;
            if (vec) {
                const uint32_t h0 = f32_to_bf16_rne(sm * acc[mt][0]) | (f32_to_bf16_rne(sm * acc[mt][1]) << 16);
                const uint32_t h1 = f32_to_bf16_rne(sm * acc[mt][2]) | (f32_to_bf16_rne(sm * acc[mt][3]) << 16);
                *reinterpret_cast<uint2*>(o) = make_uint2(h0, h1);
            } else {
                for (int r = 0; r < 4; ++r)
                    if (n0 + r < a.N) o[r] = (uint16_t)f32_to_bf16_rne(sm * acc[mt][r]);
            }
        } else {
            float* p = a.partials + ((int64_t)split * a.M + m) * a.N + n0;
            if (vec) {
                *reinterpret_cast<float4*>(p) = make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
            } else {
                for (int r = 0; r < 4; ++r)
                    if (n0 + r < a.N) p[r] = acc[mt][r];
            }
        }
    }
}

template <int MT, int D>
hipError_t launch_pdec(const PDecArgs& a, size_t lds, hipStream_t stream) {
    static bool attr_set = false;   // raise the dynamic LDS cap once per process
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)pdec_kernel<MT, D>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((pdec_kernel<MT, D>), dim3(a.groups * a.ks), dim3(256), lds, stream, a);
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
                       (int)N, (int)K, tiles, 4 * c_pad, reinterpret_cast<uint4*>(wt));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prep_s_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream, we,
                       (int)N, (int)K, tiles, c_pad, reinterpret_cast<uint32_t*>(st));
    return hipGetLastError();
}

// Decode plan on prepared weights: K splits so the split's activations fit the
// LDS budget and the grid has enough waves; D-deep ring.
GemmPlan plan_prepared(int64_t M, int64_t N, int64_t K, int ks_hint, int depth) {
    GemmPlan p{};
    p.band = 2;
    p.mt = (int)((M + 15) / 16);
    p.rt = 1;
    p.u = depth;
    const int64_t tiles = (N + 15) / 16;
    const int64_t groups = (tiles + 3) / 4;
    const int64_t c_pad = (K / 128 + 3) / 4;
    const int64_t lds_budget = 64 * 1024;
    int64_t c_max = (lds_budget / M - 16) / 512;
    if (c_max < 1) c_max = 1;
    int64_t ks = (c_pad + c_max - 1) / c_max;
    const int64_t want_waves = 2048;
    const int64_t ks_par = (want_waves + 4 * groups - 1) / (4 * groups);
    if (ks < ks_par) ks = ks_par;
    if (ks_hint > 0) ks = ks_hint < ks ? ks : ks_hint;   // a hint may only lower the split
    if (ks < (c_pad + c_max - 1) / c_max) ks = (c_pad + c_max - 1) / c_max;
    if (ks > c_pad) ks = c_pad;
    const int64_t c_per = (c_pad + ks - 1) / ks;
    p.s_per = (int)c_per;
    p.ks = (int)((c_pad + c_per - 1) / c_per);
    p.tiles = tiles;
    return p;
}

size_t prepared_lds_bytes(const GemmPlan& p, int64_t M) {
    return (size_t)(M * ((int64_t)p.s_per * 512 + 16));
}

hipError_t launch_prepared_decode(const GemmPlan& p, const uint8_t* x8, const float* xs,
                                  const uint8_t* wt, const uint8_t* st, uint16_t* out, int64_t M,
                                  int64_t N, int64_t K, void* ws, hipStream_t stream) {
    PDecArgs a{};
    a.x8 = x8; a.xs = xs;
    a.wt = reinterpret_cast<const uint4*>(wt);
    a.st = reinterpret_cast<const uint32_t*>(st);
    a.out = out;
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.c_pad = (int)((K / 128 + 3) / 4);
    a.s_pad = 4 * a.c_pad;
    a.tiles = (int)p.tiles;
    a.groups = (int)((p.tiles + 3) / 4);
    a.ks = p.ks;
    a.c_per = p.s_per;
    if (p.ks > 1)
        a.partials = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + ws_counter_bytes(p.tiles));
    const size_t lds = prepared_lds_bytes(p, M);
    hipError_t e;
    if (p.mt == 1)
        e = p.u == 4 ? launch_pdec<1, 4>(a, lds, stream) : launch_pdec<1, 3>(a, lds, stream);
    else
        e = p.u == 4 ? launch_pdec<2, 4>(a, lds, stream) : launch_pdec<2, 3>(a, lds, stream);
    if (e != hipSuccess || p.ks == 1) return e;
    return launch_splitk_reduce(a.partials, xs, M, N, p.ks, out, stream);
}

}  // namespace w4a8
