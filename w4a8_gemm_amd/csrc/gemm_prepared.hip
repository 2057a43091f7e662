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
// for LDS), fp32 partials for the reduction kernel.
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
    int tw, kw;         // tiles and K parts per workgroup
    int groups;         // workgroups per split (ceil(tiles / tw))
    int ks, c_per;      // K splits across workgroups, chunks per split
};

struct PChunk {
    uint4 w[4];
    uint32_t s;
};

__device__ __forceinline__ void pdec_load(const uint4* wp, const uint32_t* sp, int j, PChunk& c) {
#pragma unroll
    for (int u = 0; u < 4; ++u) c.w[u] = wp[(4 * j + u) * 64];
    c.s = sp[j * 64];
}

template <int MT>
__device__ __forceinline__ void pdec_compute(const uint8_t* xl, int stride, int lane, int M, int j,
                                             const PChunk& c, v4f (&acc)[MT]) {
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

constexpr int kActBatch = 8;

// activation elements q0 + u * nthreads (u < kActBatch) of the workgroup's
// [M, kr] slice, 16 bytes each
__device__ __forceinline__ void pdec_act_load(const PDecArgs& a, int kbase, int per_row, int total, int q0,
                                              int nthreads, uint4 (&v)[kActBatch]) {
#pragma unroll
    for (int u = 0; u < kActBatch; ++u) {
        const int q = q0 + u * nthreads;
        const int m = q / per_row, col = q - m * per_row;
        const int k = kbase + 16 * col;
        v[u] = (q < total && k < a.K) ? *reinterpret_cast<const uint4*>(a.x8 + (int64_t)m * a.K + k)
                                      : make_uint4(0, 0, 0, 0);
    }
}
__device__ __forceinline__ void pdec_act_store(uint8_t* xl, int stride, int per_row, int total, int q0,
                                               int nthreads, const uint4 (&v)[kActBatch]) {
#pragma unroll
    for (int u = 0; u < kActBatch; ++u) {
        const int q = q0 + u * nthreads;
        const int m = q / per_row, col = q - m * per_row;
        if (q < total) *reinterpret_cast<uint4*>(xl + m * stride + 16 * col) = v[u];
    }
}

template <int MT, int D>
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
    const int kbase = c0 * 512, kr = nch_wg * 512, stride = kr + 16;
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
    const uint32_t* sp = a.st + ((int64_t)tc * a.c_pad + c0 + jb) * 64 + lane;
    const int last = nch > 0 ? nch - 1 : 0;

    // Activations of this workgroup's K range -> LDS (columns >= K read as
    // zero), 16 bytes per thread and load, in batches of kActBatch loads per
    // thread so that their latencies overlap.  The first batch is issued
    // before the weight ring prologue: its LDS writes then wait only for these
    // (L2-resident) loads while the weight loads stay in flight.
    const int per_row = kr / 16, act_total = a.M * per_row;
    uint4 av[kActBatch];
    pdec_act_load(a, kbase, per_row, act_total, threadIdx.x, nthreads, av);
    __builtin_amdgcn_sched_barrier(0);
    PChunk ring[D];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) pdec_load(wp, sp, min(d, last), ring[d]);
    __builtin_amdgcn_sched_barrier(0);
    pdec_act_store(xl, stride, per_row, act_total, threadIdx.x, nthreads, av);
    for (int q0 = threadIdx.x + kActBatch * nthreads; q0 < act_total; q0 += kActBatch * nthreads) {
        pdec_act_load(a, kbase, per_row, act_total, q0, nthreads, av);
        pdec_act_store(xl, stride, per_row, act_total, q0, nthreads, av);
    }
    __syncthreads();

    const uint8_t* xw = xl + 512 * j0;   // this part's first activation column
    if (active) {
        for (int j = 0; j < nch; j += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                pdec_load(wp, sp, min(j + d + D - 1, last), ring[(d + D - 1) % D]);
                __builtin_amdgcn_sched_barrier(0);
                if (j + d < nch) pdec_compute<MT>(xw, stride, lane, a.M, j + d, ring[d], acc);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // add the K parts of each tile through LDS, in part order
    if (a.kw > 1) {
        __syncthreads();   // all waves are done reading activations
        float4* red = reinterpret_cast<float4*>(xl);   // [kw][tw][MT][64 lanes]
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            red[((part * a.tw + wave % a.tw) * MT + mt) * 64 + lane] =
                make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
        __syncthreads();
        if (part != 0) return;
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
    if (t >= a.tiles) return;

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
    hipLaunchKernelGGL((pdec_kernel<MT, D>), dim3(a.groups * a.ks), dim3(64 * a.tw * a.kw), lds,
                       stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// tiled band on prepared weights (M > 32): 256 weight rows x BM activation rows
// per workgroup, K in 128-wide steps through a 3-stage LDS ring.
//
// Eight waves in an NWN x NWM grid; wave tile = 16*FN weight rows x 16*FM
// activation rows of 16x16x128 MFMAs.  Every stage is filled with direct
// global -> LDS copies (global_load_lds, 1 KiB or 256 B per wave instruction, no
// registers): the 16 weight fragment blocks of the panel (lane order = MFMA
// order, read back with one conflict-free ds_read_b128 per fragment), the BM x
// 128 activation slice, whose 16-byte chunk c of row r sits at chunk position
// c ^ ((r >> 1) & 7) (so the 16 rows of a fragment read land in 16 distinct
// bank groups), and the panel's e8m0 dwords for the step's 4-step chunk.  One
// barrier per step: the wait + barrier at the top of step s makes stage s
// visible and frees stage s-1, whose slot then receives step s+2.  LDS offsets
// start at 256: a direct-to-LDS destination of address 0 would be taken for a
// null pointer by the address-space cast.
// ---------------------------------------------------------------------------

struct PfArgs {
    const uint8_t* x8;
    const float* xs;
    const uint8_t* wt;
    const uint8_t* st;
    uint16_t* out;
    int M, N, K;
    int s_pad, c_pad, tiles16;
    int tiles_m, tiles_n;
    int group_m;                // M tiles per group of the tile order
};

constexpr int kPfThreads = 512;
constexpr int kPfBN = 256;
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

template <int BM>
struct PfShape {
    static constexpr int NWM = BM >= 256 ? 4 : (BM >= 128 ? 2 : 1);
    static constexpr int NWN = 8 / NWM;
    static constexpr int FN = kPfBN / (16 * NWN);
    static constexpr int FM = BM / (16 * NWM);
    static constexpr int NS = 3;                           // ring stages
    static constexpr int WBYTES = kPfBN / 16 * 1024;      // weight blocks per stage
    static constexpr int ABYTES = BM * 128;                // activation slice
    static constexpr int STAGE = WBYTES + ABYTES;
    static constexpr int SBYTES = kPfBN / 16 * 256;        // e8m0 dwords of one 4-step chunk
    static constexpr int LDS = kPfBase + NS * STAGE + 2 * SBYTES;
    static constexpr int DMA_PER_STAGE = (kPfBN / 16) / 8 + (BM / 8) / 8;   // per wave
    static constexpr int DMA_SCALES = (kPfBN / 16) / 8;                     // per wave, per chunk
};

// Per-workgroup copy sources: one buffer descriptor per operand based at the
// workgroup's tile, per-lane offsets that stay fixed over the K steps (the
// step advance goes into the scalar offset).
template <int BM>
struct PfSrc {
    i32x4 w, x, sc;
    uint32_t w_off[2], x_off[BM / 64], s_off[2];
};

template <int BM>
__device__ __forceinline__ void pf_sources(const PfArgs& a, int tm, int tn, int wave, int lane, PfSrc<BM>& src) {
    const int t0 = tn * 16;
    const int64_t wblk = (int64_t)a.s_pad * 1024, sblk = (int64_t)a.c_pad * 256;
    src.w = make_rsrc(a.wt + t0 * wblk, (uint64_t)(a.tiles16 - t0) * wblk);
    src.sc = make_rsrc(a.st + t0 * sblk, (uint64_t)(a.tiles16 - t0) * sblk);
    src.x = make_rsrc(a.x8 + (int64_t)tm * BM * a.K, (uint64_t)(a.M - tm * BM) * a.K);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        // weight and e8m0 blocks b = wave, wave + 8 of the 16 tiles (clamped to the last tile)
        const int t = min(t0 + wave + 8 * i, a.tiles16 - 1) - t0;
        src.w_off[i] = (uint32_t)(t * wblk) + 16u * lane;
        src.s_off[i] = (uint32_t)(t * sblk) + 4u * lane;
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
// two weight blocks, then BM/64 activation row groups.
template <int BM, int J>
__device__ __forceinline__ void pf_issue_one(const PfSrc<BM>& src, uint8_t* stage, int s, int wave) {
    using S = PfShape<BM>;
    if constexpr (J < 2) {
        lds_dma16(src.w, src.w_off[J], 1024u * s, lds_addr(stage + 1024 * (wave + 8 * J)));
    } else {
        constexpr int i = J - 2;
        lds_dma16(src.x, src.x_off[i], 128u * s, lds_addr(stage + S::WBYTES + 1024 * (wave + 8 * i)));
    }
}

// e8m0 dwords of 4-step chunk c (two 256-byte blocks per wave) into `sbuf`
template <int BM>
__device__ __forceinline__ void pf_issue_scales(const PfSrc<BM>& src, uint8_t* sbuf, int c, int wave) {
#pragma unroll
    for (int i = 0; i < PfShape<BM>::DMA_SCALES; ++i)
        lds_dma4(src.sc, src.s_off[i], 256u * c, lds_addr(sbuf + 256 * (wave + 8 * i)));
}

// copies [J0, J1) of the stage
template <int BM, int J0, int J1>
__device__ __forceinline__ void pf_issue_range(const PfSrc<BM>& src, uint8_t* stage, int s, int wave) {
    if constexpr (J0 < J1) {
        pf_issue_one<BM, J0>(src, stage, s, wave);
        pf_issue_range<BM, J0 + 1, J1>(src, stage, s, wave);
    }
}

template <int BM>
__device__ __forceinline__ void pf_issue(const PfSrc<BM>& src, uint8_t* stage, int s, int wave) {
    pf_issue_range<BM, 0, PfShape<BM>::DMA_PER_STAGE>(src, stage, s, wave);
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
template <int BM, int F>
__device__ __forceinline__ void pf_copies_at(const PfSrc<BM>& src, uint8_t* nxt, int s_nxt, int wave) {
    constexpr int D = PfShape<BM>::DMA_PER_STAGE, FN = PfShape<BM>::FN;
    pf_issue_range<BM, F * D / FN, (F + 1) * D / FN>(src, nxt, s_nxt, wave);
}

template <int BM, int F>
__device__ __forceinline__ void pf_group(const uint8_t* wp, const uint32_t* sp, int sh, const v8i (&bx)[PfShape<BM>::FM],
                                         uint4& wa, uint32_t& sc, v4f (&acc)[PfShape<BM>::FN][PfShape<BM>::FM],
                                         const PfSrc<BM>& src, uint8_t* nxt, int s_nxt, int wave) {
    using S = PfShape<BM>;
    if constexpr (F < S::FN) {
        const v8i af = frag_fp4(wa);
        const int scf = (int)(sc >> sh);
        if constexpr (F + 1 < S::FN) {
            sc = sp[64 * (F + 1)];
            wa = *reinterpret_cast<const uint4*>(wp + 1024 * (F + 1));
        }
        pf_copies_at<BM, F>(src, nxt, s_nxt, wave);
#pragma unroll
        for (int h = 0; h < S::FM; ++h) acc[F][h] = mfma16<0>(af, bx[h], acc[F][h], scf);
        __builtin_amdgcn_sched_barrier(0);
        pf_group<BM, F + 1>(wp, sp, sh, bx, wa, sc, acc, src, nxt, s_nxt, wave);
    }
}

template <int BM>
__device__ __forceinline__ void pf_compute(const uint8_t* st, int s, int wn, int wm, int lane,
                                           v4f (&acc)[PfShape<BM>::FN][PfShape<BM>::FM],
                                           const uint8_t* sbuf,
                                           const PfSrc<BM>& src, uint8_t* nxt, int s_nxt, int wave) {
    using S = PfShape<BM>;
    const int g = lane >> 4;
    const uint8_t* ws = st;
    const uint8_t* as = st + S::WBYTES;
    const uint32_t* ss = reinterpret_cast<const uint32_t*>(sbuf);
    // activation fragments of the wave's FM column tiles, then the weight
    // fragments one at a time against all of them, the next one's LDS read
    // issued before the current one's products
    v8i bx[S::FM];
#pragma unroll
    for (int h = 0; h < S::FM; ++h) {
        const int r = wm * 16 * S::FM + 16 * h + (lane & 15);
        const int sw = (r >> 1) & 7;
        const uint8_t* rowp = as + 128 * r;
        bx[h] = frag_fp8(*reinterpret_cast<const uint4*>(rowp + 16 * (g ^ sw)),
                         *reinterpret_cast<const uint4*>(rowp + 16 * ((4 + g) ^ sw)));
    }
    const uint8_t* wp = ws + 1024 * (wn * S::FN) + 16 * lane;
    const uint32_t* sp = ss + 64 * (wn * S::FN) + lane;
    uint32_t sc = sp[0];
    uint4 wa = *reinterpret_cast<const uint4*>(wp);
    pf_group<BM, 0>(wp, sp, 8 * (s & 3), bx, wa, sc, acc, src, nxt, s_nxt, wave);
}


// Three-stage ring, copies issued two steps ahead; e8m0 chunks (one per four
// steps) in two buffers of their own.  Per step s: wait for the copies of
// step s (those of step s + 1 may stay in flight), barrier (stage visible to
// all waves; the stage read in step s - 1 is free), issue the e8m0 chunk that
// starts at step s + 2 (if any), then compute, with the copies for step s + 2
// into the free stage issued between the products.  In issue order the
// copies of step u are: [e8m0 chunk u/4 if u % 4 == 0] [weights, activations].
template <int BM>
__global__ __launch_bounds__(kPfThreads) void pf_kernel(PfArgs a) {
    using S = PfShape<BM>;
    constexpr int D = S::DMA_PER_STAGE, DS = S::DMA_SCALES;
    __shared__ __attribute__((aligned(16))) uint8_t lds[S::LDS];
    const int total = a.tiles_m * a.tiles_n;
    const int per_xcd = (total + 7) >> 3;
    const int T = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (T >= total) return;
    const int gm = a.group_m;
    const int group = T / (gm * a.tiles_n);
    const int first_m = group * gm;
    const int gsize = min(a.tiles_m - first_m, gm);
    const int rem = T % (gm * a.tiles_n);
    const int tm = first_m + rem % gsize, tn = rem / gsize;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wn = wave % S::NWN, wm = wave / S::NWN;

    v4f acc[S::FN][S::FM];
#pragma unroll
    for (int f = 0; f < S::FN; ++f)
#pragma unroll
        for (int h = 0; h < S::FM; ++h) acc[f][h] = v4f{0.f, 0.f, 0.f, 0.f};

    const int steps = a.K >> 7;
    uint8_t* const base = lds + kPfBase;
    uint8_t* const sbase = base + S::NS * S::STAGE;
    PfSrc<BM> src;
    pf_sources<BM>(a, tm, tn, wave, lane, src);
    // prologue: step 0 (with e8m0 chunk 0) and step 1 (repeating step 0 when K has one step)
    pf_issue_scales<BM>(src, sbase, 0, wave);
    pf_issue<BM>(src, base, 0, wave);
    pf_issue<BM>(src, base + S::STAGE, min(1, steps - 1), wave);
    int cur = 0, nxt = 2 * S::STAGE;       // stage offsets of steps s and s + 2
    for (int s = 0; s < steps; ++s) {
        // opaque to the optimiser: stage addresses are formed per step from a
        // few lane bases and immediate offsets instead of being unrolled and
        // hoisted into dozens of live registers
        asm volatile("" : "+s"(cur), "+s"(nxt));
        if (((s + 1) & 3) == 0 && s + 1 < steps) wait_vmcnt<D + DS>();
        else wait_vmcnt<D>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");     // no LDS access moves across the barrier
        const int u = s + 2;
        if ((u & 3) == 0 && u < steps) pf_issue_scales<BM>(src, sbase + ((u >> 2) & 1) * S::SBYTES, u >> 2, wave);
        // copies for step s + 2; in the last two steps they repeat the last
        // step into the free stage, which is never read again (no branch in
        // the product sequence)
        pf_compute<BM>(base + cur, s, wn, wm, lane, acc, sbase + ((s >> 2) & 1) * S::SBYTES, src, base + nxt,
                       min(u, steps - 1), wave);
        cur = cur == 2 * S::STAGE ? 0 : cur + S::STAGE;
        nxt = nxt == 2 * S::STAGE ? 0 : nxt + S::STAGE;
    }
    // the repeated copies of the last steps may still be landing: drain them
    // before the workgroup's LDS is released
    wait_vmcnt<0>();
    const int g = lane >> 4;

    // epilogue: lane holds rows n0..n0+3 of column m in every 16x16 tile
    const bool vec = (a.N & 3) == 0;
#pragma unroll
    for (int h = 0; h < S::FM; ++h) {
        const int m = tm * BM + wm * 16 * S::FM + 16 * h + (lane & 15);
        if (m >= a.M) continue;
        const float sm = a.xs[m];
#pragma unroll
        for (int f = 0; f < S::FN; ++f) {
            const int n0 = tn * kPfBN + (wn * S::FN + f) * 16 + 4 * g;
            if (n0 >= a.N) continue;
            uint16_t* o = a.out + (int64_t)m * a.N + n0;
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

template <int BM>
hipError_t launch_pf(const PfArgs& a, hipStream_t stream) {
    const int total = a.tiles_m * a.tiles_n;
    const int grid = (total + 7) / 8 * 8;
    hipLaunchKernelGGL((pf_kernel<BM>), dim3(grid), dim3(kPfThreads), 0, stream, a);
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

// Decode plan on prepared weights: plan fields rt = tiles per workgroup, kw =
// K parts per tile, ks = K splits across workgroups, s_per = chunks per split,
// u = ring depth.
static void prepared_shape(int64_t M, int64_t N, int64_t K, int* tw, int* kw, int* ks, int* c_per) {
    const int64_t tiles = (N + 15) / 16;
    const int64_t c_pad = (K / 128 + 3) / 4;
    const int64_t act_budget = 80 * 1024;          // activations resident in LDS per workgroup
    // K splits across workgroups only when the activations do not fit
    int64_t c_max = (act_budget / M - 16) / 512;
    if (c_max < 1) c_max = 1;
    int64_t s = (c_pad + c_max - 1) / c_max;
    int64_t cp = (c_pad + s - 1) / s;
    s = (c_pad + cp - 1) / cp;
    // tiles per workgroup: enough activation reuse (the L2 -> LDS copies,
    // M*K per workgroup, at most about a quarter of the weight bytes), at most 4
    int64_t t_w = (M + 3) / 4;
    if (t_w < 1) t_w = 1;
    if (t_w > 4) t_w = 4;
    // K parts per tile (measured on gfx950: two for wide layers, four for
    // narrow ones), at most 16 waves per group
    int64_t k_w = tiles * s >= 1024 ? 2 : 4;
    if (k_w > cp) k_w = cp;
    if (k_w > 16 / t_w) k_w = 16 / t_w;
    if (k_w < 1) k_w = 1;
    *tw = (int)t_w;
    *kw = (int)k_w;
    *ks = (int)s;
    *c_per = (int)cp;
}

GemmPlan plan_prepared(int64_t M, int64_t N, int64_t K, int ks_hint, int depth) {
    GemmPlan p{};
    p.band = 2;
    p.mt = (int)((M + 15) / 16);
    int tw, kw, ks, cp;
    prepared_shape(M, N, K, &tw, &kw, &ks, &cp);
    if (ks_hint > 0) {   // tuning: ks_hint encodes kw (K parts per tile)
        kw = ks_hint;
        if (kw * tw > 16) kw = 16 / tw;
        if (kw > cp) kw = cp;
    }
    p.rt = tw;
    p.kw = kw;
    p.u = depth;
    p.ks = ks;
    p.s_per = cp;
    p.tiles = (N + 15) / 16;
    return p;
}

size_t prepared_lds_bytes(const GemmPlan& p, int64_t M) {
    const size_t act = (size_t)(M * ((int64_t)p.s_per * 512 + 16));
    const size_t red = (size_t)p.kw * p.rt * p.mt * 64 * 16;
    return act > red ? act : red;
}

hipError_t launch_prepared_tiled(const uint8_t* x8, const float* xs, const uint8_t* wt,
                                 const uint8_t* st, uint16_t* out, int64_t M, int64_t N, int64_t K,
                                 hipStream_t stream) {
    PfArgs a{};
    a.x8 = x8; a.xs = xs; a.wt = wt; a.st = st; a.out = out;
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.c_pad = (int)((K / 128 + 3) / 4);
    a.s_pad = 4 * a.c_pad;
    a.tiles16 = (int)((N + 15) / 16);
    a.tiles_n = (int)((N + kPfBN - 1) / kPfBN);
    if ((M + 63) / 64 * (int64_t)a.tiles_n > (int64_t)INT32_MAX - 8) return hipErrorInvalidValue;
    a.group_m = 8;
    if (M <= 64) {
        a.tiles_m = (int)((M + 63) / 64);
        return launch_pf<64>(a, stream);
    }
    if (M <= 128) {
        a.tiles_m = (int)((M + 127) / 128);
        return launch_pf<128>(a, stream);
    }
    a.tiles_m = (int)((M + 255) / 256);
    return launch_pf<256>(a, stream);
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
    a.tw = p.rt;
    a.kw = p.kw;
    a.groups = (int)((p.tiles + p.rt - 1) / p.rt);
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
