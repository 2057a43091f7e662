// gemm_int4.hip -- int4 group-128 symmetric W4A8 GEMM and its load-time preparation.
//
// "radiance_autoround.py": AutoGPTQ layout, qweight [K/8, N] int32 with nibble j
// of word i holding k = 8i + j; scales [K/128, N] fp16; qzeros all 0x77777777
// (zero point 8, so code c means c - 8); the reference dequantizes
// (c - 8) * scale[k/128, n] and multiplies by the fp8 activations times their
// per-token scale.  process_weights_after_loading rejects asymmetric zeros and
// transposes the weight to [N, K/8] so that one row of N is contiguous.
//
// c - 8 (-8..7) is exact in e4m3, so the product runs on the fp8 x fp8 matrix
// cores (V_MFMA_SCALE_*_F8F6F4 with unit scales); each 128-wide K group is one
// MFMA (16x16x128, decode) or two (32x32x64, prefill) into a fresh accumulator,
// which is then added into the output accumulator times the group's fp16 scale
// (fp32 arithmetic).  The nibble -> e4m3 byte map is an 8-entry byte table per
// sign half applied with v_perm_b32.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kFmtFp8 = 0;
constexpr int kUnitScale = 127;

// 32 codes (4 words, k = 32 consecutive) -> fp8 fragment of the same k order
__device__ __forceinline__ v8i int4x32_frag(uint4 q) {
    const uint2 a = int4x8_to_e4m3(q.x), b = int4x8_to_e4m3(q.y);
    const uint2 c = int4x8_to_e4m3(q.z), d = int4x8_to_e4m3(q.w);
    v8i r = {(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y, (int)d.x, (int)d.y};
    return r;
}

__device__ __forceinline__ v4f mfma16_f8(v8i a, v8i b, v4f c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kFmtFp8, kFmtFp8, 0, kUnitScale, 0,
                                                            kUnitScale);
}
__device__ __forceinline__ v16f mfma32_f8(v8i a, v8i b, v16f c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, kFmtFp8, kFmtFp8, 0, kUnitScale, 0,
                                                           kUnitScale);
}

// ---------------------------------------------------------------------------
// load-time preparation
// ---------------------------------------------------------------------------

__global__ void count_asym_kernel(const uint32_t* __restrict__ qz, int64_t n, uint32_t* bad) {
    uint32_t c = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        c += (qz[i] != 0x77777777u) ? 1u : 0u;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if ((threadIdx.x & 63) == 0 && c) atomicAdd(bad, c);
}

// [R, C] int32 -> [C, R] through a 64x64 LDS tile (padded against bank conflicts)
__global__ __launch_bounds__(256) void transpose_kernel(const int32_t* __restrict__ in, int64_t R,
                                                        int64_t C, int32_t* __restrict__ out) {
    __shared__ int32_t t[64][65];
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < 64; i += 4) {
        const int64_t r = r0 + i, c = c0 + tx;
        if (r < R && c < C) t[i][tx] = in[r * C + c];
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
        const int64_t c = c0 + i, r = r0 + tx;
        if (r < R && c < C) out[c * R + r] = t[tx][i];
    }
}

// ---------------------------------------------------------------------------
// decode band (M <= 64): as the MXFP4 decode kernel, one 128-group per MFMA
// and U groups per prefetched chunk.  Weight lane (n, g) holds k = 32g .. 32g+31
// of the group (16 bytes of codes at 64G + 16g, so a load instruction reads 64
// contiguous bytes of 16 rows), expanded to 32 e4m3 bytes; the activation lane
// (m, g) holds the same 32 activation bytes (the fp8 operand's byte j < 16 sits
// at MFMA slot 16g + j and byte 16 + j at slot 64 + 16g + j, identically for
// both operands).  The lane's four output rows n0..n0+3 take their group scales
// from one 8-byte load.  Split K goes through fp32 partials that the row
// block's last split to arrive adds in place (sk_arrive / sk_reduce).
// ---------------------------------------------------------------------------

constexpr int kDecThreads = 256;

struct I4DecArgs {
    const uint8_t* x8;
    const float* xs;
    const int32_t* qw;
    const uint16_t* sc;
    uint16_t* out;
    float* partials;
    uint32_t* counters;   // ks > 1: one arrival counter per row block
    int sk_inplace;       // ks > 1: the last split reduces (else the reduction kernel does)
    int M, N, K;
    int ks, s_per, tiles;
};

template <int MT, int RT, int U>
struct I4Chunk {
    uint4 w[RT][U];
    uint2 s[RT][U];
    uint4 x[MT][U][2];
};

template <int MT, int RT, int U>
__device__ __forceinline__ void i4_load(const I4DecArgs& a, int lane, const int* rows, int row0,
                                        int grp, I4Chunk<MT, RT, U>& c) {
    const int g = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int32_t* wr = a.qw + (int64_t)rows[rt] * (a.K >> 3) + 16 * (int64_t)grp + 4 * g;
        const int n0 = min(row0 + rt * 16 + 4 * g, a.N - 4);   // N % 8 == 0, so n0..n0+3 in range
#pragma unroll
        for (int u = 0; u < U; ++u) {
            c.w[rt][u] = *reinterpret_cast<const uint4*>(wr + 16 * u);
            c.s[rt][u] = *reinterpret_cast<const uint2*>(a.sc + (int64_t)(grp + u) * a.N + n0);
        }
    }
    // columns m >= M load row M-1 (never stored): unconditional loads
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = min(mt * 16 + (lane & 15), a.M - 1);
        const uint8_t* xr = a.x8 + (int64_t)m * a.K + 128 * (int64_t)grp + 32 * g;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            c.x[mt][u][0] = *reinterpret_cast<const uint4*>(xr + 128 * u);
            c.x[mt][u][1] = *reinterpret_cast<const uint4*>(xr + 128 * u + 16);
        }
    }
}

template <int MT, int RT, int U>
__device__ __forceinline__ void i4_compute(const I4Chunk<MT, RT, U>& c, v4f (&acc)[RT][MT]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const v8i aw = int4x32_frag(c.w[rt][u]);
            const float s[4] = {f16_to_f32(c.s[rt][u].x & 0xFFFFu), f16_to_f32(c.s[rt][u].x >> 16),
                                f16_to_f32(c.s[rt][u].y & 0xFFFFu), f16_to_f32(c.s[rt][u].y >> 16)};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const v8i bx = {(int)c.x[mt][u][0].x, (int)c.x[mt][u][0].y, (int)c.x[mt][u][0].z,
                                (int)c.x[mt][u][0].w, (int)c.x[mt][u][1].x, (int)c.x[mt][u][1].y,
                                (int)c.x[mt][u][1].z, (int)c.x[mt][u][1].w};
                const v4f t = mfma16_f8(aw, bx, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[rt][mt][r] = __builtin_fmaf(s[r], t[r], acc[rt][mt][r]);
            }
        }
    }
}

template <int MT, int RT, int U>
__global__ __launch_bounds__(kDecThreads) void i4_decode_kernel(I4DecArgs a) {
    const int tile = blockIdx.x % a.tiles;
    const int split = blockIdx.x / a.tiles;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int row0 = tile * (4 * RT * 16) + wave * (RT * 16);
    int rows[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) rows[rt] = min(row0 + rt * 16 + (lane & 15), a.N - 1);

    const int groups = a.K >> 7;
    const int s0 = split * a.s_per;
    const int s1 = min(groups, s0 + a.s_per);
    v4f acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = v4f{0.f, 0.f, 0.f, 0.f};

    int grp = s0;
    const int nchunks = s1 > s0 ? (s1 - s0) / U : 0;
    if (nchunks > 0) {   // two register sets in turn, loads fenced from the MFMAs
        I4Chunk<MT, RT, U> ca, cb;
        i4_load<MT, RT, U>(a, lane, rows, row0, s0, ca);
        int c = 1;
        for (; c + 1 < nchunks; c += 2) {
            i4_load<MT, RT, U>(a, lane, rows, row0, s0 + c * U, cb);
            __builtin_amdgcn_sched_barrier(0);
            i4_compute<MT, RT, U>(ca, acc);
            __builtin_amdgcn_sched_barrier(0);
            i4_load<MT, RT, U>(a, lane, rows, row0, s0 + (c + 1) * U, ca);
            __builtin_amdgcn_sched_barrier(0);
            i4_compute<MT, RT, U>(cb, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (c < nchunks) {
            i4_load<MT, RT, U>(a, lane, rows, row0, s0 + c * U, cb);
            __builtin_amdgcn_sched_barrier(0);
            i4_compute<MT, RT, U>(ca, acc);
            __builtin_amdgcn_sched_barrier(0);
            i4_compute<MT, RT, U>(cb, acc);
        } else {
            i4_compute<MT, RT, U>(ca, acc);
        }
        grp = s0 + nchunks * U;
    }
    for (; grp < s1; ++grp) {
        I4Chunk<MT, RT, 1> one;
        i4_load<MT, RT, 1>(a, lane, rows, row0, grp, one);
        i4_compute<MT, RT, 1>(one, acc);
    }

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int n0 = row0 + rt * 16 + 4 * g;
        if (n0 >= a.N) continue;   // N % 8 == 0: n0 < N means n0..n0+3 < N
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mt * 16 + (lane & 15);
            if (m >= a.M) continue;
            if (a.ks == 1) {
                const float sm = a.xs[m];
                const uint32_t h0 = f32_to_bf16_rne(sm * acc[rt][mt][0]) | (f32_to_bf16_rne(sm * acc[rt][mt][1]) << 16);
                const uint32_t h1 = f32_to_bf16_rne(sm * acc[rt][mt][2]) | (f32_to_bf16_rne(sm * acc[rt][mt][3]) << 16);
                *reinterpret_cast<uint2*>(a.out + (int64_t)m * a.N + n0) = make_uint2(h0, h1);
            } else {
                sk_put4(sk_rsrc(a.partials), 4u * (uint32_t)(((int64_t)split * a.M + m) * a.N + n0),
                        acc[rt][mt][0], acc[rt][mt][1], acc[rt][mt][2], acc[rt][mt][3]);
            }
        }
    }
    if (a.ks > 1 && a.sk_inplace) {
        // K split: the row block's last split to arrive adds the partials
        __shared__ uint32_t last_flag;
        if (sk_arrive(a.counters + tile, a.ks, &last_flag))
            sk_reduce(a.partials, a.xs, a.M, a.N, a.ks, tile * (4 * RT * 16), min(a.N, (tile + 1) * (4 * RT * 16)),
                      a.out, threadIdx.x, kDecThreads);
    }
}


// ---------------------------------------------------------------------------
// prefill band: 128x128 tiles, one 128-group per K step, weights expanded to
// e4m3 while staging into LDS, 2x2 waves of 2x2 32x32x64 MFMA tiles; each
// step's two MFMAs per tile go into a fresh accumulator that is added in times
// the group scale of its row.
// ---------------------------------------------------------------------------

constexpr int kPreThreads = 256;
constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kRowStride = kBK + 16;  // padded e4m3 row
constexpr int kABytes = kBN * kRowStride;
constexpr int kBBytes = kBM * kRowStride;
constexpr int kSBytes = kBN * 4;      // group scales as fp32
constexpr int kStageBytes = kABytes + kBBytes + kSBytes;

struct I4PreArgs {
    const uint8_t* x8;
    const float* xs;
    const int32_t* qw;
    const uint16_t* sc;
    uint16_t* out;
    int M, N, K;
    int tiles_m, tiles_n;
};

struct I4PreRegs {
    uint4 a[2];
    uint4 b[4];
    float s;
};

__device__ __forceinline__ void i4_pre_load(const I4PreArgs& a, int m0, int n0, int grp, I4PreRegs& r) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = t + i * kPreThreads;
        const int row = c >> 2, part = c & 3;
        const int n = min(n0 + row, a.N - 1);
        r.a[i] = *reinterpret_cast<const uint4*>(a.qw + (int64_t)n * (a.K >> 3) + 16 * (int64_t)grp + 4 * part);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = t + i * kPreThreads;
        const int row = c >> 3, part = c & 7;
        const int m = min(m0 + row, a.M - 1);
        r.b[i] = *reinterpret_cast<const uint4*>(a.x8 + (int64_t)m * a.K + 128 * (int64_t)grp + 16 * part);
    }
    if (t < kBN) r.s = f16_to_f32(a.sc[(int64_t)grp * a.N + min(n0 + t, a.N - 1)]);
}

__device__ __forceinline__ void i4_pre_store(uint8_t* stage, const I4PreRegs& r) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = t + i * kPreThreads;
        const int row = c >> 2, part = c & 3;  // 16 B of codes = 32 k = 32 e4m3 bytes
        const v8i f = int4x32_frag(r.a[i]);
        uint4* p = reinterpret_cast<uint4*>(stage + row * kRowStride + 32 * part);
        p[0] = make_uint4((uint32_t)f[0], (uint32_t)f[1], (uint32_t)f[2], (uint32_t)f[3]);
        p[1] = make_uint4((uint32_t)f[4], (uint32_t)f[5], (uint32_t)f[6], (uint32_t)f[7]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = t + i * kPreThreads;
        const int row = c >> 3, part = c & 7;
        *reinterpret_cast<uint4*>(stage + kABytes + row * kRowStride + 16 * part) = r.b[i];
    }
    if (t < kBN) reinterpret_cast<float*>(stage + kABytes + kBBytes)[t] = r.s;
}

__global__ __launch_bounds__(kPreThreads) void i4_prefill_kernel(I4PreArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];
    const int total = a.tiles_m * a.tiles_n;
    const int per_xcd = (total + 7) >> 3;
    const int T = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (T >= total) return;
    const int group = T / (8 * a.tiles_n);
    const int first_m = group * 8;
    const int gsize = min(a.tiles_m - first_m, 8);
    const int rem = T % (8 * a.tiles_n);
    const int tm = first_m + rem % gsize, tn = rem / gsize;
    const int m0 = tm * kBM, n0 = tn * kBN;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wn = wave >> 1, wm = wave & 1;
    const int g = lane >> 5, r32 = lane & 31;

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int groups = a.K >> 7;
    I4PreRegs regs;
    i4_pre_load(a, m0, n0, 0, regs);
    i4_pre_store(smem, regs);
    __syncthreads();
    for (int grp = 0; grp < groups; ++grp) {
        uint8_t* cur = smem + (grp & 1) * kStageBytes;
        uint8_t* nxt = smem + ((grp + 1) & 1) * kStageBytes;
        const bool more = grp + 1 < groups;
        if (more) i4_pre_load(a, m0, n0, grp + 1, regs);
        const uint8_t* As = cur;
        const uint8_t* Bs = cur + kABytes;
        const float* Ss = reinterpret_cast<const float*>(cur + kABytes + kBBytes);
        v16f tmp[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) tmp[i][j][e] = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            v8i af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint8_t* p = As + (wn * 64 + i * 32 + r32) * kRowStride + 64 * u + 16 * g;
                const uint4 lo = *reinterpret_cast<const uint4*>(p), hi = *reinterpret_cast<const uint4*>(p + 32);
                v8i f = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                af[i] = f;
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint8_t* p = Bs + (wm * 64 + j * 32 + r32) * kRowStride + 64 * u + 16 * g;
                const uint4 lo = *reinterpret_cast<const uint4*>(p), hi = *reinterpret_cast<const uint4*>(p + 32);
                v8i f = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                bf[j] = f;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) tmp[i][j] = mfma32_f8(af[i], bf[j], tmp[i][j]);
        }
        // scale rows n = 8q + 4g + rr of each 32-row tile
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const float s = Ss[wn * 64 + i * 32 + 8 * q + 4 * g + rr];
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j][4 * q + rr] = __builtin_fmaf(s, tmp[i][j][4 * q + rr], acc[i][j][4 * q + rr]);
                }
            }
        }
        if (more) i4_pre_store(nxt, regs);
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = m0 + wm * 64 + j * 32 + r32;
        if (m >= a.M) continue;
        const float sm = a.xs[m];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * 64 + i * 32 + 8 * q + 4 * g;
                uint16_t* o = a.out + (int64_t)m * a.N + n;
                const float v0 = sm * acc[i][j][4 * q + 0], v1 = sm * acc[i][j][4 * q + 1];
                const float v2 = sm * acc[i][j][4 * q + 2], v3 = sm * acc[i][j][4 * q + 3];
                if (n + 3 < a.N && (a.N & 3) == 0) {
                    const uint32_t h0 = f32_to_bf16_rne(v0) | (f32_to_bf16_rne(v1) << 16);
                    const uint32_t h1 = f32_to_bf16_rne(v2) | (f32_to_bf16_rne(v3) << 16);
                    *reinterpret_cast<uint2*>(o) = make_uint2(h0, h1);
                } else {
                    const float v[4] = {v0, v1, v2, v3};
                    for (int r = 0; r < 4; ++r)
                        if (n + r < a.N) o[r] = (uint16_t)f32_to_bf16_rne(v[r]);
                }
            }
        }
    }
}

template <int MT, int RT, int U>
hipError_t launch_i4dec(const I4DecArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((i4_decode_kernel<MT, RT, U>), dim3(a.tiles * a.ks), dim3(kDecThreads), 0, stream, a);
    return hipGetLastError();
}

template <int MT, int RT>
hipError_t launch_i4dec_u(const I4DecArgs& a, int u, hipStream_t stream) {
    switch (u) {
        case 1: return launch_i4dec<MT, RT, 1>(a, stream);
        case 2: return launch_i4dec<MT, RT, 2>(a, stream);
        default: return launch_i4dec<MT, RT, 4>(a, stream);
    }
}

template <int MT>
hipError_t launch_i4dec_rt(const I4DecArgs& a, int rt, int u, hipStream_t stream) {
    switch (rt) {
        case 1: return launch_i4dec_u<MT, 1>(a, u, stream);
        case 2: return launch_i4dec_u<MT, 2>(a, u, stream);
        default: return launch_i4dec_u<MT, 4>(a, u, stream);
    }
}

}  // namespace

GemmPlan plan_int4(int64_t M, int64_t N, int64_t K) {
    if (M > 64) {
        GemmPlan p{};
        p.band = 1;
        return p;
    }
    const int mt = (int)((M + 15) / 16);
    const int rt = mt >= 3 ? 1 : 2;
    const int u = mt >= 2 ? 2 : 4;
    const int64_t tiles = (N + 4 * rt * 16 - 1) / (4 * rt * 16);
    const int64_t ks = (512 + tiles - 1) / tiles;
    return make_decode_plan(M, N, K, rt, u, (int)ks);
}

hipError_t launch_int4_check_transpose(const int32_t* qw_kn, const int32_t* qzeros, int64_t N,
                                       int64_t K, int32_t* qw_nk, uint32_t* bad_count,
                                       hipStream_t stream) {
    if (qzeros) {
        const int64_t nz = (K / 128) * (N / 8);
        const int64_t want = (nz + 255) / 256;
        const int grid = (int)(want < 1024 ? (want > 0 ? want : 1) : 1024);
        hipLaunchKernelGGL(count_asym_kernel, dim3(grid), dim3(256), 0, stream,
                           reinterpret_cast<const uint32_t*>(qzeros), nz, bad_count);
        return hipGetLastError();
    }
    const int64_t R = K / 8, C = N;
    hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64)),
                       dim3(256), 0, stream, qw_kn, R, C, qw_nk);
    return hipGetLastError();
}

hipError_t launch_int4_gemm(const GemmPlan& p, const uint8_t* x8, const float* xs,
                            const int32_t* qw_nk, const uint16_t* scales, uint16_t* out,
                            int64_t M, int64_t N, int64_t K, void* ws, hipStream_t stream) {
    if (p.band == 1) {
        I4PreArgs a{x8, xs, qw_nk, scales, out, (int)M, (int)N, (int)K,
                    (int)((M + kBM - 1) / kBM), (int)((N + kBN - 1) / kBN)};
        const int total = a.tiles_m * a.tiles_n;
        const int grid = (total + 7) / 8 * 8;
        hipLaunchKernelGGL(i4_prefill_kernel, dim3(grid), dim3(kPreThreads), 0, stream, a);
        return hipGetLastError();
    }
    I4DecArgs a{};
    a.x8 = x8; a.xs = xs; a.qw = qw_nk; a.sc = scales; a.out = out;
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.ks = p.ks; a.s_per = p.s_per; a.tiles = (int)p.tiles;
    if (p.ks > 1) {
        a.counters = reinterpret_cast<uint32_t*>(ws);
        a.partials = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + ws_counter_bytes(p.tiles));
        a.sk_inplace = sk_inplace_fits(p.ks, M, N) ? 1 : 0;
    }
    hipError_t e;
    switch (p.mt) {
        case 1: e = launch_i4dec_rt<1>(a, p.rt, p.u, stream); break;
        case 2: e = launch_i4dec_rt<2>(a, p.rt, p.u, stream); break;
        case 3: e = launch_i4dec_rt<3>(a, p.rt, p.u, stream); break;
        default: e = launch_i4dec_rt<4>(a, p.rt, p.u, stream); break;
    }
    if (e != hipSuccess || p.ks == 1 || a.sk_inplace) return e;
    return launch_splitk_reduce(a.partials, xs, M, N, p.ks, out, stream);
}

}  // namespace w4a8
