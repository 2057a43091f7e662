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
// columns (MT tiles of 16), and the workgroup one K split.  A 512-wide K chunk
// is 4 MFMAs; in MFMA u, weight lane (row, g) holds 32-block 4g+u of the chunk,
// so the lane's four weight fragments are one contiguous 64-byte run and its
// four e8m0 bytes one aligned dword (opsel u picks the byte).  The activation
// lane (m, g) then needs 16-byte halves of blocks 4(g/2)+u and 8+4(g/2)+u,
// half g%2, which it reads from L2 (activations are small and shared).
// A K remainder of fewer than 4 steps runs 128 wide with the hardware order.
// ===========================================================================

constexpr int kDecThreads = 256;

struct DecArgs {
    const uint8_t* x8;
    const float* xs;
    const uint8_t* wq;
    const uint8_t* we;
    uint16_t* out;
    uint32_t* counters;
    float* partials;
    int M, N, K;
    int ks;        // K splits
    int s_per;     // 128-wide steps per split
    int tiles;     // row blocks (4 * RT * 16 rows each)
};

template <int MT>
__device__ __forceinline__ void load_act_chunk(const DecArgs& a, int lane, int64_t kbyte, int u,
                                               v8i* bx) {
    const int g = lane >> 4;
    const int aoff = 128 * (g >> 1) + 16 * (g & 1) + 32 * u;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + (lane & 15);
        uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
        if (m < a.M) {
            const uint8_t* p = a.x8 + (int64_t)m * a.K + kbyte + aoff;
            lo = *reinterpret_cast<const uint4*>(p);
            hi = *reinterpret_cast<const uint4*>(p + 256);
        }
        bx[mt] = frag_fp8(lo, hi);
    }
}

// one 128-wide step in the hardware order, with K-tail masking (K % 32 == 0)
template <int MT, int RT, bool ALIGNED_SCALE>
__device__ __forceinline__ void dec_step(const DecArgs& a, int lane, const int* rows, int s,
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
    (void)ALIGNED_SCALE;
}

template <int RT>
struct WChunk {
    uint4 q[RT][4];
    uint32_t sc[RT];
};

template <int RT>
__device__ __forceinline__ void load_w_chunk(const DecArgs& a, int lane, const int* rows, int s,
                                             WChunk<RT>& c) {
    const int g = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const uint4* p = reinterpret_cast<const uint4*>(a.wq + (int64_t)rows[rt] * (a.K >> 1) +
                                                        64 * (int64_t)s + 64 * g);
#pragma unroll
        for (int u = 0; u < 4; ++u) c.q[rt][u] = p[u];
        c.sc[rt] = *reinterpret_cast<const uint32_t*>(a.we + (int64_t)rows[rt] * (a.K >> 5) + 4 * s + 4 * g);
    }
}

template <int MT, int RT>
__device__ __forceinline__ void dec_chunk(const DecArgs& a, int lane, int s, const WChunk<RT>& c,
                                          v4f (&acc)[RT][MT]) {
    const int64_t kbyte = 128 * (int64_t)s;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        v8i bx[MT];
        load_act_chunk<MT>(a, lane, kbyte, u, bx);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const v8i aw = frag_fp4(c.q[rt][u]);
            const int sc = (int)c.sc[rt];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (u == 0) acc[rt][mt] = mfma16<0>(aw, bx[mt], acc[rt][mt], sc);
                if (u == 1) acc[rt][mt] = mfma16<1>(aw, bx[mt], acc[rt][mt], sc);
                if (u == 2) acc[rt][mt] = mfma16<2>(aw, bx[mt], acc[rt][mt], sc);
                if (u == 3) acc[rt][mt] = mfma16<3>(aw, bx[mt], acc[rt][mt], sc);
            }
        }
    }
}

template <int MT, int RT, bool K128>
__global__ __launch_bounds__(kDecThreads) void mx_decode_kernel(DecArgs a) {
    // XCD-aware order: all K splits of a row block land on the same XCD
    // (workgroups are dealt round-robin over the 8 XCDs), so the partial sums
    // a last-arriving workgroup reads were written through its own L2.
    const int b = blockIdx.x;
    const int xcd = b & 7, li = b >> 3;
    const int split = li % a.ks;
    const int tile = (li / a.ks) * 8 + xcd;
    if (tile >= a.tiles) return;

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
    if (K128 && s + 4 <= s1) {
        WChunk<RT> cur;
        load_w_chunk<RT>(a, lane, rows, s, cur);
        for (; s + 4 <= s1; s += 4) {
            WChunk<RT> nxt;
            const bool more = s + 8 <= s1;
            if (more) load_w_chunk<RT>(a, lane, rows, s + 4, nxt);
            dec_chunk<MT, RT>(a, lane, s, cur, acc);
            if (more) cur = nxt;
        }
    }
    for (; s < s1; ++s) dec_step<MT, RT, K128>(a, lane, rows, s, acc);

    // ---------------- epilogue ----------------
    const int g = lane >> 4;
    if (a.ks == 1) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int n0 = row0 + rt * 16 + 4 * g;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = mt * 16 + (lane & 15);
                if (m >= a.M) continue;
                const float sm = a.xs[m];
                uint16_t* o = a.out + (int64_t)m * a.N + n0;
                if (n0 + 3 < a.N && (a.N & 3) == 0) {
                    const uint32_t h0 = f32_to_bf16_rne(sm * acc[rt][mt][0]) | (f32_to_bf16_rne(sm * acc[rt][mt][1]) << 16);
                    const uint32_t h1 = f32_to_bf16_rne(sm * acc[rt][mt][2]) | (f32_to_bf16_rne(sm * acc[rt][mt][3]) << 16);
                    *reinterpret_cast<uint2*>(o) = make_uint2(h0, h1);
                } else {
                    for (int r = 0; r < 4; ++r)
                        if (n0 + r < a.N) o[r] = (uint16_t)f32_to_bf16_rne(sm * acc[rt][mt][r]);
                }
            }
        }
        return;
    }

    // split K: publish this split's partial sums, then the last arrival reduces
    // all splits in fixed order 0..ks-1 (bitwise deterministic) and resets the
    // counter for the next call.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int n0 = row0 + rt * 16 + 4 * g;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mt * 16 + (lane & 15);
            if (m >= a.M) continue;
            float* p = a.partials + ((int64_t)split * a.M + m) * a.N + n0;
            if (n0 + 3 < a.N && (a.N & 3) == 0) {
                *reinterpret_cast<float4*>(p) = make_float4(acc[rt][mt][0], acc[rt][mt][1], acc[rt][mt][2], acc[rt][mt][3]);
            } else {
                for (int r = 0; r < 4; ++r)
                    if (n0 + r < a.N) p[r] = acc[rt][mt][r];
            }
        }
    }
    __threadfence();
    __syncthreads();
    __shared__ int last;
    if (threadIdx.x == 0) {
        const uint32_t prev = atomicAdd(&a.counters[tile], 1u);
        last = (prev == (uint32_t)(a.ks - 1));
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int n0 = row0 + rt * 16 + 4 * g;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mt * 16 + (lane & 15);
            if (m >= a.M) continue;
            const float sm = a.xs[m];
            uint16_t* o = a.out + (int64_t)m * a.N + n0;
            if (n0 + 3 < a.N && (a.N & 3) == 0) {
                float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
                for (int j = 0; j < a.ks; ++j) {
                    const float4 v = *reinterpret_cast<const float4*>(a.partials + ((int64_t)j * a.M + m) * a.N + n0);
                    t.x = t.x + v.x;
                    t.y = t.y + v.y;
                    t.z = t.z + v.z;
                    t.w = t.w + v.w;
                }
                const uint32_t h0 = f32_to_bf16_rne(sm * t.x) | (f32_to_bf16_rne(sm * t.y) << 16);
                const uint32_t h1 = f32_to_bf16_rne(sm * t.z) | (f32_to_bf16_rne(sm * t.w) << 16);
                *reinterpret_cast<uint2*>(o) = make_uint2(h0, h1);
            } else {
                for (int r = 0; r < 4; ++r) {
                    if (n0 + r >= a.N) continue;
                    float t = 0.f;
                    for (int j = 0; j < a.ks; ++j) t = t + a.partials[((int64_t)j * a.M + m) * a.N + n0 + r];
                    o[r] = (uint16_t)f32_to_bf16_rne(sm * t);
                }
            }
        }
    }
    if (threadIdx.x == 0) a.counters[tile] = 0u;
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

template <int MT, int RT>
hipError_t launch_dec(const DecArgs& a, bool k128, hipStream_t stream) {
    const int grid = ((a.tiles + 7) / 8) * 8 * a.ks;
    if (k128)
        hipLaunchKernelGGL((mx_decode_kernel<MT, RT, true>), dim3(grid), dim3(kDecThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((mx_decode_kernel<MT, RT, false>), dim3(grid), dim3(kDecThreads), 0, stream, a);
    return hipGetLastError();
}

template <int RT>
hipError_t launch_dec_rt(const DecArgs& a, int mt, bool k128, hipStream_t stream) {
    switch (mt) {
        case 1: return launch_dec<1, RT>(a, k128, stream);
        case 2: return launch_dec<2, RT>(a, k128, stream);
        case 3: return launch_dec<3, RT>(a, k128, stream);
        default: return launch_dec<4, RT>(a, k128, stream);
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// plans
// ---------------------------------------------------------------------------

static int steps_per_split(int64_t steps, int64_t tiles, bool k128) {
    // aim for about 4 workgroups (16 waves) per CU over 256 CUs
    const int64_t target = 1024;
    int64_t sp = (steps * tiles + target - 1) / target;
    if (sp < 1) sp = 1;
    if (k128) sp = (sp + 3) / 4 * 4;
    if (sp > steps) sp = steps;
    return (int)sp;
}

GemmPlan plan_mxfp4(int64_t M, int64_t N, int64_t K) {
    GemmPlan p{};
    if (M > 64) {
        p.band = 1;
        return p;
    }
    p.band = 0;
    p.mt = (int)((M + 15) / 16);
    p.rt = 4;
    const int64_t rows_per_tile = 4 * p.rt * 16;
    p.tiles = (N + rows_per_tile - 1) / rows_per_tile;
    const int64_t steps = (K + 127) / 128;
    p.s_per = steps_per_split(steps, p.tiles, K % 128 == 0);
    p.ks = (int)((steps + p.s_per - 1) / p.s_per);
    return p;
}

size_t plan_workspace_bytes(const GemmPlan& p, int64_t M, int64_t N) {
    if (p.band != 0 || p.ks <= 1) return 0;
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
    a.ks = p.ks;
    a.s_per = p.s_per;
    a.tiles = (int)p.tiles;
    if (p.ks > 1) {
        a.counters = reinterpret_cast<uint32_t*>(ws);
        a.partials = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + ws_counter_bytes(p.tiles));
    }
    const bool k128 = (K % 128) == 0;
    switch (p.rt) {
        case 1: return launch_dec_rt<1>(a, p.mt, k128, stream);
        case 2: return launch_dec_rt<2>(a, p.mt, k128, stream);
        default: return launch_dec_rt<4>(a, p.mt, k128, stream);
    }
}

}  // namespace w4a8
