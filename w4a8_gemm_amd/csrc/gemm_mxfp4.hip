// gemm_mxfp4.hip -- block-scaled W4A8 GEMM on gfx950 matrix cores.
//
//   out[m,n] = bf16_rne( s_m * sum_k e4m3(x8[m,k]) * e2m1(w[n,k]) * 2^(E[n,k/32]-127) )
//
// "vllm-radiance (MXFP4)", How the MXFP4 path works, The W4A8 fp8-WMMA kernel:
// fp8 activations against e2m1 weights whose e8m0 scale is folded into the
// product, a decode tiling for small M with split-K whose last-arriving
// workgroup reduces the partial sums, and a separate tiled prefill band.
//
// On CDNA4 the e8m0 fold is native: V_MFMA_SCALE_F32_{16X16X128,32X32X64}_F8F6F4
// take the e2m1 weight fragment (format 4) with one e8m0 byte per lane and
// 32-wide K block, and the e4m3 activation fragment (format 0) with unit scale
// (127).  The weight is the A operand (rows n), the activations the B operand
// (columns m), so each lane's accumulators hold 4 consecutive n of one m and the
// epilogue stores 8-byte bf16 runs.
//
// Operand layout of these instructions (measured on gfx950):
//   fp4 operand, lane (row r, group g):  k = 32g + j for nibble j (16 bytes)
//   fp8 operand, 16x16x128, lane (r, g): bytes 0-15 -> k = 16g + j,
//                                        bytes 16-31 -> k = 64 + 16g + j
//   fp8 operand, 32x32x64, lane (r, g):  bytes 0-15 -> k = 16g + j,
//                                        bytes 16-31 -> k = 32 + 16g + j
//   scale of (row r, 32-block b) is lane 16b + r (16x16) or 32b + r (32x32),
//   byte `opsel` of that lane's scale register.
// Because the contraction is a sum over k, each MFMA's 32-wide K blocks may be
// any 32-blocks of the weight as long as both operands and the scale agree; the
// kernels use that to give every weight lane a contiguous run of bytes.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

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
template <int OPSEL>
__device__ __forceinline__ v16f mfma32(v8i a_fp4, v8i b_fp8, v16f c, int scale_a) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a_fp4, b_fp8, c, kFmtFp4, kFmtFp8, OPSEL,
                                                           scale_a, 0, kUnitScale);
}

// ===========================================================================
// Decode band (M <= 64): weights streamed from HBM straight into registers.
//
// Workgroup = 4 waves; wave w owns RT*16 consecutive weight rows and all M
// columns (MT tiles of 16); the grid covers row blocks x K splits.  The K range
// of a split is walked in chunks of U 128-wide steps, one MFMA per step and
// 16-row tile, in the instruction's own K order: weight lane (n, g) of step t
// holds bytes 64t + 16g .. +16 of row n, so each load instruction reads 64
// contiguous bytes of 16 rows; its e8m0 byte is byte g of the row's dword for
// the step (shifted down, opsel 0); activation lane (m, g) holds bytes
// 128t + 16g and 128t + 64 + 16g of row m (L2 resident, shared by all waves).
// The whole next chunk (weights, scales, activations) is issued before the
// current chunk's MFMAs, so one chunk of loads is always in flight per wave.
// With more than one K split each split writes fp32 partial sums through to the
// device's coherence point, and the row block's last split to arrive adds
// them in split order (bitwise deterministic; sk_arrive / sk_reduce).
// K % 128 != 0 runs one masked step at a time (U = 1).
// ===========================================================================

constexpr int kDecThreads = 256;

struct DecArgs {
    const uint8_t* x8;
    const float* xs;
    const uint8_t* wq;
    const uint8_t* we;
    uint16_t* out;
    float* partials;
    uint32_t* counters;   // ks > 1: one arrival counter per row block
    int sk_inplace;       // ks > 1: the last split reduces (else the reduction kernel does)
    int M, N, K;
    int ks;        // K splits
    int s_per;     // 128-wide steps per split
    int tiles;     // row blocks (4 * RT * 16 rows each)
};

template <int MT, int RT, int U>
struct DecChunk {
    uint4 w[RT][U];
    uint32_t s[RT][U];
    uint4 x[MT][U][2];
};

template <int MT, int RT, int U>
__device__ __forceinline__ void dec_load(const DecArgs& a, int lane, const int* rows, int s,
                                         DecChunk<MT, RT, U>& c) {
    const int g = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const uint8_t* wr = a.wq + (int64_t)rows[rt] * (a.K >> 1) + 64 * (int64_t)s + 16 * g;
        const uint8_t* er = a.we + (int64_t)rows[rt] * (a.K >> 5) + 4 * (int64_t)s;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            c.w[rt][u] = *reinterpret_cast<const uint4*>(wr + 64 * u);
            c.s[rt][u] = *reinterpret_cast<const uint32_t*>(er + 4 * u);
        }
    }
    // columns m >= M load row M-1 (their outputs are never stored): every load
    // is unconditional, so the wait before the MFMAs covers only this chunk
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = min(mt * 16 + (lane & 15), a.M - 1);
        const uint8_t* xr = a.x8 + (int64_t)m * a.K + 128 * (int64_t)s + 16 * g;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            c.x[mt][u][0] = *reinterpret_cast<const uint4*>(xr + 128 * u);
            c.x[mt][u][1] = *reinterpret_cast<const uint4*>(xr + 128 * u + 64);
        }
    }
}

template <int MT, int RT, int U>
__device__ __forceinline__ void dec_compute(int lane, const DecChunk<MT, RT, U>& c,
                                            v4f (&acc)[RT][MT]) {
    const int sh = 8 * (lane >> 4);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const v8i aw = frag_fp4(c.w[rt][u]);
            const int sc = (int)(c.s[rt][u] >> sh);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[rt][mt] = mfma16<0>(aw, frag_fp8(c.x[mt][u][0], c.x[mt][u][1]), acc[rt][mt], sc);
        }
    }
}

// one 128-wide step with K-tail masking (any K % 32 == 0)
template <int MT, int RT>
__device__ __forceinline__ void dec_step_masked(const DecArgs& a, int lane, const int* rows, int s,
                                                v4f (&acc)[RT][MT]) {
    const int g = lane >> 4;
    const int kb = 4 * s;                 // first 32-block of the step
    const int kblocks = a.K >> 5;
    const bool wvalid = kb + g < kblocks;
    const bool p1valid = kb + (g >> 1) < kblocks;
    const bool p2valid = kb + 2 + (g >> 1) < kblocks;
    v8i bx[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + (lane & 15);
        uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
        if (m < a.M) {
            const uint8_t* p = a.x8 + (int64_t)m * a.K + 128 * (int64_t)s + 16 * g;
            if (p1valid) lo = *reinterpret_cast<const uint4*>(p);
            if (p2valid) hi = *reinterpret_cast<const uint4*>(p + 64);
        }
        bx[mt] = frag_fp8(lo, hi);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        uint4 q = make_uint4(0, 0, 0, 0);
        int sc = kUnitScale;
        if (wvalid) {
            q = *reinterpret_cast<const uint4*>(a.wq + (int64_t)rows[rt] * (a.K >> 1) + 64 * (int64_t)s + 16 * g);
            sc = a.we[(int64_t)rows[rt] * kblocks + kb + g];
        }
        const v8i aw = frag_fp4(q);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = mfma16<0>(aw, bx[mt], acc[rt][mt], sc);
    }
}

template <int MT, int RT, int U, bool K128>
__global__ __launch_bounds__(kDecThreads) void mx_decode_kernel(DecArgs a) {
    const int tile = blockIdx.x % a.tiles;
    const int split = blockIdx.x / a.tiles;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row0 = tile * (4 * RT * 16) + wave * (RT * 16);
    int rows[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) rows[rt] = min(row0 + rt * 16 + (lane & 15), a.N - 1);

    const int steps = (a.K + 127) >> 7;
    const int s0 = split * a.s_per;
    const int s1 = min(steps, s0 + a.s_per);

    v4f acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = v4f{0.f, 0.f, 0.f, 0.f};

    int s = s0;
    if (K128) {
        // software pipeline: the loop body always issues the next chunk's loads
        // before the current chunk's MFMAs (straight-line, so the wait before
        // the MFMAs only covers the current chunk)
        // Two register sets used in turn (no copies); scheduling barriers keep
        // the compiler from sinking a prefetch next to its use.
        const int nchunks = s1 > s0 ? (s1 - s0) / U : 0;
        if (nchunks > 0) {
            DecChunk<MT, RT, U> ca, cb;
            dec_load<MT, RT, U>(a, lane, rows, s0, ca);
            int c = 1;
            for (; c + 1 < nchunks; c += 2) {
                dec_load<MT, RT, U>(a, lane, rows, s0 + c * U, cb);
                __builtin_amdgcn_sched_barrier(0);
                dec_compute<MT, RT, U>(lane, ca, acc);
                __builtin_amdgcn_sched_barrier(0);
                dec_load<MT, RT, U>(a, lane, rows, s0 + (c + 1) * U, ca);
                __builtin_amdgcn_sched_barrier(0);
                dec_compute<MT, RT, U>(lane, cb, acc);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (c < nchunks) {
                dec_load<MT, RT, U>(a, lane, rows, s0 + c * U, cb);
                __builtin_amdgcn_sched_barrier(0);
                dec_compute<MT, RT, U>(lane, ca, acc);
                __builtin_amdgcn_sched_barrier(0);
                dec_compute<MT, RT, U>(lane, cb, acc);
            } else {
                dec_compute<MT, RT, U>(lane, ca, acc);
            }
            s = s0 + nchunks * U;
        }
        for (; s < s1; ++s) {
            DecChunk<MT, RT, 1> one;
            dec_load<MT, RT, 1>(a, lane, rows, s, one);
            dec_compute<MT, RT, 1>(lane, one, acc);
        }
    } else {
        for (; s < s1; ++s) dec_step_masked<MT, RT>(a, lane, rows, s, acc);
    }

    // epilogue: lane holds rows n0..n0+3 (n0 = tile row + 4g) of column m
    const int g = lane >> 4;
    const bool vec = (a.N & 3) == 0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int n0 = row0 + rt * 16 + 4 * g;
        if (n0 >= a.N) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mt * 16 + (lane & 15);
            if (m >= a.M) continue;
            if (a.ks == 1) {
                const float sm = a.xs[m];
                uint16_t* o = a.out + (int64_t)m * a.N + n0;
                if (vec) {
                    const uint32_t h0 = f32_to_bf16_rne(sm * acc[rt][mt][0]) | (f32_to_bf16_rne(sm * acc[rt][mt][1]) << 16);
                    const uint32_t h1 = f32_to_bf16_rne(sm * acc[rt][mt][2]) | (f32_to_bf16_rne(sm * acc[rt][mt][3]) << 16);
                    *reinterpret_cast<uint2*>(o) = make_uint2(h0, h1);
                } else {
                    for (int r = 0; r < 4; ++r)
                        if (n0 + r < a.N) o[r] = (uint16_t)f32_to_bf16_rne(sm * acc[rt][mt][r]);
                }
            } else if (vec) {
                sk_put4(sk_rsrc(a.partials), 4u * (uint32_t)(((int64_t)split * a.M + m) * a.N + n0),
                        acc[rt][mt][0], acc[rt][mt][1], acc[rt][mt][2], acc[rt][mt][3]);
            } else {
                float* p = a.partials + ((int64_t)split * a.M + m) * a.N + n0;
                for (int r = 0; r < 4; ++r)
                    if (n0 + r < a.N) sk_put(p + r, acc[rt][mt][r]);
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

// out[m, n] = bf16(s_m * sum_{j < ks} partials[j, m, n]), j in increasing order
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partials,
                                                            const float* __restrict__ xs, int M,
                                                            int N, int ks, uint16_t* __restrict__ out) {
    const int64_t total = (int64_t)M * N;
    const int64_t plane = total;
    if ((N & 3) == 0) {
        const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
        if (i4 >= total) return;
        const int m = (int)(i4 / N);
        float4 t = *reinterpret_cast<const float4*>(partials + i4);
        for (int j = 1; j < ks; ++j) {
            const float4 v = *reinterpret_cast<const float4*>(partials + (int64_t)j * plane + i4);
            t.x = t.x + v.x;
            t.y = t.y + v.y;
            t.z = t.z + v.z;
            t.w = t.w + v.w;
        }
        const float sm = xs ? xs[m] : 1.0f;   // no token scale: the scales were inside the products
        const uint32_t h0 = f32_to_bf16_rne(sm * t.x) | (f32_to_bf16_rne(sm * t.y) << 16);
        const uint32_t h1 = f32_to_bf16_rne(sm * t.z) | (f32_to_bf16_rne(sm * t.w) << 16);
        *reinterpret_cast<uint2*>(out + i4) = make_uint2(h0, h1);
    } else {
        const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
        if (i >= total) return;
        float t = partials[i];
        for (int j = 1; j < ks; ++j) t = t + partials[(int64_t)j * plane + i];
        out[i] = (uint16_t)f32_to_bf16_rne((xs ? xs[i / N] : 1.0f) * t);
    }
}


// ===========================================================================
// Prefill band (M > 64): 128x128 output tile per workgroup, K in steps of 128
// staged through LDS (double buffered, one barrier per step).  Four waves in a
// 2x2 grid each own 64 (n) x 64 (m) outputs = 2x2 tiles of the 32x32x64 MFMA.
// In MFMA u (0, 1) of a step, weight lane (n, g) holds 32-block 2g+u, i.e. 16
// bytes at offset 32g+16u of the row's 64-byte step slice, and its e8m0 bytes
// are bytes 2g, 2g+1 of the row's scale dword (shifted down, opsel u); the
// activation lane (m, g) holds halves g of blocks u and 2+u.  Rows of both LDS
// tiles are padded by 16 bytes so the 16-byte fragment reads of 16 consecutive
// rows fall in distinct banks.
// ===========================================================================

constexpr int kPreThreads = 256;
constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kAStride = kBK / 2 + 16;  // weight tile row: 64 B + pad
constexpr int kBStride = kBK + 16;      // activation tile row: 128 B + pad
constexpr int kABytes = kBN * kAStride;
constexpr int kBBytes = kBM * kBStride;
constexpr int kSBytes = kBN * 4;
constexpr int kStageBytes = kABytes + kBBytes + kSBytes;

struct PreArgs {
    const uint8_t* x8;
    const float* xs;
    const uint8_t* wq;
    const uint8_t* we;
    uint16_t* out;
    int M, N, K;
    int tiles_m, tiles_n;
};

struct PreRegs {
    uint4 a[2];   // weight chunks
    uint4 b[4];   // activation chunks
    uint32_t s;   // scale dword (threads < kBN)
};

__device__ __forceinline__ void pre_load(const PreArgs& a, int m0, int n0, int step, PreRegs& r) {
    const int t = threadIdx.x;
    const int k0 = step * kBK;
    const int kblocks = a.K >> 5;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = t + i * kPreThreads;
        const int row = c >> 2, part = c & 3;
        const int n = min(n0 + row, a.N - 1);
        const bool ok = (k0 / 32 + part) < kblocks;  // 16 B of e2m1 = one 32-block
        r.a[i] = ok ? *reinterpret_cast<const uint4*>(a.wq + (int64_t)n * (a.K >> 1) + k0 / 2 + 16 * part)
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = t + i * kPreThreads;
        const int row = c >> 3, part = c & 7;
        const int m = min(m0 + row, a.M - 1);
        const bool ok = (k0 / 32 + part / 2) < kblocks;
        r.b[i] = ok ? *reinterpret_cast<const uint4*>(a.x8 + (int64_t)m * a.K + k0 + 16 * part)
                    : make_uint4(0, 0, 0, 0);
    }
    if (t < kBN) {
        const int n = min(n0 + t, a.N - 1);
        const uint8_t* p = a.we + (int64_t)n * kblocks + k0 / 32;
        uint32_t s = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t byte = (k0 / 32 + q < kblocks) ? (uint32_t)p[q] : (uint32_t)kUnitScale;
            s |= byte << (8 * q);
        }
        r.s = s;
    }
}

__device__ __forceinline__ void pre_store(uint8_t* stage, const PreRegs& r) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = t + i * kPreThreads;
        const int row = c >> 2, part = c & 3;
        *reinterpret_cast<uint4*>(stage + row * kAStride + 16 * part) = r.a[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = t + i * kPreThreads;
        const int row = c >> 3, part = c & 7;
        *reinterpret_cast<uint4*>(stage + kABytes + row * kBStride + 16 * part) = r.b[i];
    }
    if (t < kBN) *reinterpret_cast<uint32_t*>(stage + kABytes + kBBytes + 4 * t) = r.s;
}

__global__ __launch_bounds__(kPreThreads) void mx_prefill_kernel(PreArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];
    // XCD-aware order: each XCD takes a contiguous range of tile ids, and tile
    // ids walk groups of 8 m-tiles down one weight panel at a time, so the
    // weight and activation panels in flight on one XCD stay in its L2.
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

    const int steps = (a.K + kBK - 1) / kBK;
    PreRegs regs;
    pre_load(a, m0, n0, 0, regs);
    pre_store(smem, regs);
    __syncthreads();

    for (int step = 0; step < steps; ++step) {
        uint8_t* cur = smem + (step & 1) * kStageBytes;
        uint8_t* nxt = smem + ((step + 1) & 1) * kStageBytes;
        const bool more = step + 1 < steps;
        if (more) pre_load(a, m0, n0, step + 1, regs);

        const uint8_t* As = cur;
        const uint8_t* Bs = cur + kABytes;
        const uint32_t* Ss = reinterpret_cast<const uint32_t*>(cur + kABytes + kBBytes);
        int sc[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) sc[i] = (int)(Ss[wn * 64 + i * 32 + r32] >> (16 * g));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            v8i af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint8_t* p = As + (wn * 64 + i * 32 + r32) * kAStride + 32 * g + 16 * u;
                af[i] = frag_fp4(*reinterpret_cast<const uint4*>(p));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint8_t* p = Bs + (wm * 64 + j * 32 + r32) * kBStride + 32 * u + 16 * g;
                bf[j] = frag_fp8(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 64));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (u == 0) acc[i][j] = mfma32<0>(af[i], bf[j], acc[i][j], sc[i]);
                    else acc[i][j] = mfma32<1>(af[i], bf[j], acc[i][j], sc[i]);
                }
        }
        if (more) pre_store(nxt, regs);
        __syncthreads();
    }

    // epilogue: lane holds m = r32 of each 32-column tile and, for q = 0..3,
    // rows n = 8q + 4g + {0..3} of each 32-row tile
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
hipError_t launch_dec(const DecArgs& a, bool k128, hipStream_t stream) {
    const int grid = a.tiles * a.ks;
    if (k128)
        hipLaunchKernelGGL((mx_decode_kernel<MT, RT, U, true>), dim3(grid), dim3(kDecThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((mx_decode_kernel<MT, RT, 1, false>), dim3(grid), dim3(kDecThreads), 0, stream, a);
    return hipGetLastError();
}

template <int MT, int RT>
hipError_t launch_dec_u(const DecArgs& a, int u, bool k128, hipStream_t stream) {
    switch (u) {
        case 1: return launch_dec<MT, RT, 1>(a, k128, stream);
        case 2: return launch_dec<MT, RT, 2>(a, k128, stream);
        default: return launch_dec<MT, RT, 4>(a, k128, stream);
    }
}

template <int MT>
hipError_t launch_dec_rt(const DecArgs& a, int rt, int u, bool k128, hipStream_t stream) {
    switch (rt) {
        case 1: return launch_dec_u<MT, 1>(a, u, k128, stream);
        case 2: return launch_dec_u<MT, 2>(a, u, k128, stream);
        default: return launch_dec_u<MT, 4>(a, u, k128, stream);
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// plans
// ---------------------------------------------------------------------------

// Decode plan: weight rows per wave (16*rt), steps per chunk (u) and K splits
// (ks).  Splits are sized so the grid holds about `target` workgroups; each
// split covers a whole number of chunks.
GemmPlan make_decode_plan(int64_t M, int64_t N, int64_t K, int rt, int u, int ks_hint) {
    GemmPlan p{};
    p.band = 0;
    p.mt = (int)((M + 15) / 16);
    p.rt = rt;
    p.u = (K % 128 == 0) ? u : 1;
    const int64_t rows_per_tile = 4 * (int64_t)p.rt * 16;
    p.tiles = (N + rows_per_tile - 1) / rows_per_tile;
    const int64_t steps = (K + 127) / 128;
    int64_t ks = ks_hint;
    if (ks < 1) ks = 1;
    if (ks > steps) ks = steps;
    int64_t sp = (steps + ks - 1) / ks;
    sp = (sp + p.u - 1) / p.u * p.u;
    p.s_per = (int)sp;
    p.ks = (int)((steps + sp - 1) / sp);
    return p;
}

GemmPlan plan_mxfp4(int64_t M, int64_t N, int64_t K) {
    if (M > 64) {
        GemmPlan p{};
        p.band = 1;
        return p;
    }
    // measured on gfx950 (gate_up 34816x5120, down_proj 5120x17408): one wave
    // per 32 rows with 512-wide chunks for M <= 16, 64 rows otherwise; K split
    // into pieces of about 1-1.5k
    const int mt = (int)((M + 15) / 16);
    const int rt = mt == 1 ? 2 : 4;
    const int u = (mt >= 3 && N < 16384) ? 2 : 4;
    const int64_t steps = (K + 127) / 128;
    const int64_t tiles = (N + 4 * rt * 16 - 1) / (4 * rt * 16);
    int64_t ks = tiles >= 256 ? (steps + 9) / 10 : (steps + 11) / 12;
    if (mt == 1 && tiles >= 256) ks = (steps + 7) / 8;
    return make_decode_plan(M, N, K, rt, u, (int)ks);
}

size_t plan_workspace_bytes(const GemmPlan& p, int64_t M, int64_t N) {
    if (p.band == 1 || p.ks <= 1) return 0;
    return ws_counter_bytes(p.tiles) + (size_t)p.ks * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_mxfp4_gemm(const GemmPlan& p, const uint8_t* x8, const float* xs,
                             const uint8_t* wq, const uint8_t* we, uint16_t* out, int64_t M,
                             int64_t N, int64_t K, void* ws, hipStream_t stream) {
    if (p.band == 1) {
        PreArgs a{x8, xs, wq, we, out, (int)M, (int)N, (int)K,
                  (int)((M + kBM - 1) / kBM), (int)((N + kBN - 1) / kBN)};
        const int total = a.tiles_m * a.tiles_n;
        const int grid = (total + 7) / 8 * 8;
        hipLaunchKernelGGL(mx_prefill_kernel, dim3(grid), dim3(kPreThreads), 0, stream, a);
        return hipGetLastError();
    }
    DecArgs a{};
    a.x8 = x8; a.xs = xs; a.wq = wq; a.we = we; a.out = out;
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.ks = p.ks; a.s_per = p.s_per; a.tiles = (int)p.tiles;
    if (p.ks > 1) {
        a.counters = reinterpret_cast<uint32_t*>(ws);
        a.partials = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + ws_counter_bytes(p.tiles));
        a.sk_inplace = sk_inplace_fits(p.ks, M, N) ? 1 : 0;
    }
    const bool k128 = (K % 128) == 0;
    hipError_t e;
    switch (p.mt) {
        case 1: e = launch_dec_rt<1>(a, p.rt, p.u, k128, stream); break;
        case 2: e = launch_dec_rt<2>(a, p.rt, p.u, k128, stream); break;
        case 3: e = launch_dec_rt<3>(a, p.rt, p.u, k128, stream); break;
        default: e = launch_dec_rt<4>(a, p.rt, p.u, k128, stream); break;
    }
    if (e != hipSuccess || p.ks == 1 || a.sk_inplace) return e;
    return launch_splitk_reduce(a.partials, xs, M, N, p.ks, out, stream);
}

hipError_t launch_splitk_reduce(const float* partials, const float* xs, int64_t M, int64_t N,
                                int ks, uint16_t* out, hipStream_t stream) {
    const int64_t items = (N % 4 == 0) ? M * N / 4 : M * N;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0,
                       stream, partials, xs, (int)M, (int)N, ks, out);
    return hipGetLastError();
}

}  // namespace w4a8
