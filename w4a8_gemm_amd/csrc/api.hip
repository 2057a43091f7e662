// api.hip -- the C ABI of libw4a8 (declared in include/w4a8.h).
//
// Every entry point validates its arguments on the host before it enqueues
// anything, then launches the kernels on the caller's stream.  No device memory
// is allocated or freed here; nothing is printed; no environment is read.
#include <math.h>

#include <mutex>

#include "w4a8_internal.h"

using namespace w4a8;

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kDecodeMaxM = 64;

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline w4a8_status hip_status(hipError_t e) { return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP; }

w4a8_status check_gemm_common(const void* x8, const void* xs, const void* w, void* out,
                              int64_t M, int64_t N, int64_t K) {
    if (!x8 || !xs || !w || !out) return W4A8_ERR_INVALID_ARG;
    if (M < 1 || N < 1 || K < 1 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return W4A8_ERR_INVALID_ARG;
    if (!aligned(x8, 16) || !aligned(xs, 4) || !aligned(w, 16) || !aligned(out, 8))
        return W4A8_ERR_INVALID_ARG;
    return W4A8_OK;
}

w4a8_status check_workspace(size_t need, void* ws, size_t ws_bytes) {
    if (need == 0) return W4A8_OK;
    if (!ws || ws_bytes < need || !aligned(ws, 256)) return W4A8_ERR_WORKSPACE;
    return W4A8_OK;
}

}  // namespace

extern "C" {

w4a8_status w4a8_requant_nvfp4_to_mxfp4(const uint8_t* d_nv_packed, const uint8_t* d_nv_scale,
                                        const int64_t* h_part_rows, const float* h_part_divisor,
                                        int n_parts, int64_t K, w4a8_exp_mode mode,
                                        int64_t row_chunk, uint8_t* d_mx_packed,
                                        uint8_t* d_mx_e8m0, double* d_err_stats, void* stream) {
    if (!d_nv_packed || !d_nv_scale || !h_part_rows || !h_part_divisor || !d_mx_packed || !d_mx_e8m0)
        return W4A8_ERR_INVALID_ARG;
    if (n_parts < 1 || row_chunk < 0 || K < 1 || K > kMaxDim) return W4A8_ERR_INVALID_ARG;
    if (mode != W4A8_EXP_OCP && mode != W4A8_EXP_NOCLIP && mode != W4A8_EXP_MSE)
        return W4A8_ERR_INVALID_ARG;
    if (K % 32 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    if (!aligned(d_nv_packed, 16) || !aligned(d_mx_packed, 16) || !aligned(d_nv_scale, 2) ||
        (d_err_stats && !aligned(d_err_stats, 8)))
        return W4A8_ERR_INVALID_ARG;
    for (int p = 0; p < n_parts; ++p) {
        const float gd = h_part_divisor[p];
        if (h_part_rows[p] < 0 || h_part_rows[p] > kMaxDim) return W4A8_ERR_INVALID_ARG;
        if (!(gd > 0.0f) || !isfinite(gd)) return W4A8_ERR_INVALID_ARG;
    }
    hipStream_t s = as_stream(stream);
    if (d_err_stats) {
        const hipError_t e = launch_fill_zero_f64(d_err_stats, 2 * (int64_t)n_parts, s);
        if (e != hipSuccess) return W4A8_ERR_HIP;
    }
    // Every partition and every row chunk in one launch (groups of up to
    // requant_max_parts() partitions): the passes of row_chunk rows change no
    // output, each block being encoded on its own, so they are not separate
    // launches.
    const int group = requant_max_parts();
    int64_t r0 = 0;
    for (int p0 = 0; p0 < n_parts; p0 += group) {
        const int n = n_parts - p0 < group ? n_parts - p0 : group;
        int64_t blocks[64];
        int64_t rows = 0;
        for (int i = 0; i < n; ++i) {
            blocks[i] = h_part_rows[p0 + i] * (K / 32);
            rows += h_part_rows[p0 + i];
        }
        const hipError_t e = launch_requant(d_nv_packed + r0 * (K / 2), d_nv_scale + r0 * (K / 16), blocks,
                                            h_part_divisor + p0, n, (int)mode, d_mx_packed + r0 * (K / 2),
                                            d_mx_e8m0 + r0 * (K / 32), d_err_stats ? d_err_stats + 2 * p0 : nullptr,
                                            s);
        if (e != hipSuccess) return W4A8_ERR_HIP;
        r0 += rows;
    }
    return W4A8_OK;
}

// bf16 or fp8-per-channel weight [rows, K] -> MXFP4, one launch
static w4a8_status quant_load(const void* d_w, const float* d_row_scale, bool fp8, int64_t rows, int64_t K,
                              w4a8_exp_mode mode, uint8_t* d_mx_packed, uint8_t* d_mx_e8m0,
                              double* d_err_stats, void* stream) {
    if (!d_w || (fp8 && !d_row_scale) || !d_mx_packed || !d_mx_e8m0) return W4A8_ERR_INVALID_ARG;
    if (rows < 0 || rows > kMaxDim || K < 1 || K > kMaxDim) return W4A8_ERR_INVALID_ARG;
    if (mode != W4A8_EXP_OCP && mode != W4A8_EXP_NOCLIP && mode != W4A8_EXP_MSE) return W4A8_ERR_INVALID_ARG;
    if (K % 32 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    if (rows * (K / 32) >= ((int64_t)1 << 32)) return W4A8_ERR_UNSUPPORTED_SHAPE;   // 32-bit block index
    if (!aligned(d_w, 16) || !aligned(d_mx_packed, 16) || (fp8 && !aligned(d_row_scale, 4)) ||
        (d_err_stats && !aligned(d_err_stats, 8)))
        return W4A8_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    if (d_err_stats && launch_fill_zero_f64(d_err_stats, 2, s) != hipSuccess) return W4A8_ERR_HIP;
    if (fp8)
        return hip_status(launch_quant_fp8ch(static_cast<const uint8_t*>(d_w), d_row_scale, rows, K, (int)mode,
                                             d_mx_packed, d_mx_e8m0, d_err_stats, s));
    return hip_status(launch_quant_bf16(static_cast<const uint16_t*>(d_w), rows, K, (int)mode, d_mx_packed,
                                        d_mx_e8m0, d_err_stats, s));
}

w4a8_status w4a8_quant_bf16_to_mxfp4(const uint16_t* d_w_bf16, int64_t rows, int64_t K, w4a8_exp_mode mode,
                                     uint8_t* d_mx_packed, uint8_t* d_mx_e8m0, double* d_err_stats,
                                     void* stream) {
    return quant_load(d_w_bf16, nullptr, false, rows, K, mode, d_mx_packed, d_mx_e8m0, d_err_stats, stream);
}

w4a8_status w4a8_quant_fp8ch_to_mxfp4(const uint8_t* d_w_e4m3, const float* d_row_scale, int64_t rows,
                                      int64_t K, w4a8_exp_mode mode, uint8_t* d_mx_packed, uint8_t* d_mx_e8m0,
                                      double* d_err_stats, void* stream) {
    return quant_load(d_w_e4m3, d_row_scale, true, rows, K, mode, d_mx_packed, d_mx_e8m0, d_err_stats,
                      stream);
}

// ---- the load-time encoders writing fragment order directly ----
static w4a8_status check_prepared_out(int64_t rows, int64_t K, w4a8_exp_mode mode, uint8_t* d_w_prepared,
                                      uint8_t* d_s_prepared) {
    if (!d_w_prepared || !d_s_prepared) return W4A8_ERR_INVALID_ARG;
    if (rows < 0 || rows > kMaxDim || K < 1 || K > kMaxDim) return W4A8_ERR_INVALID_ARG;
    if (mode != W4A8_EXP_OCP && mode != W4A8_EXP_NOCLIP && mode != W4A8_EXP_MSE) return W4A8_ERR_INVALID_ARG;
    if (K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    if (!aligned(d_w_prepared, 16) || !aligned(d_s_prepared, 4)) return W4A8_ERR_INVALID_ARG;
    return W4A8_OK;
}

w4a8_status w4a8_requant_nvfp4_to_mxfp4_prepared(const uint8_t* d_nv_packed, const uint8_t* d_nv_scale,
                                                 const int64_t* h_part_rows, const float* h_part_divisor,
                                                 int n_parts, int64_t K, w4a8_exp_mode mode,
                                                 uint8_t* d_w_prepared, uint8_t* d_s_prepared, void* stream) {
    if (!d_nv_packed || !d_nv_scale || !h_part_rows || !h_part_divisor) return W4A8_ERR_INVALID_ARG;
    if (n_parts < 1 || n_parts > requant_max_parts()) return W4A8_ERR_INVALID_ARG;
    if (!aligned(d_nv_packed, 16) || !aligned(d_nv_scale, 2)) return W4A8_ERR_INVALID_ARG;
    int64_t rows = 0, blocks[64];
    for (int p = 0; p < n_parts; ++p) {
        const float gd = h_part_divisor[p];
        if (h_part_rows[p] < 0 || h_part_rows[p] > kMaxDim) return W4A8_ERR_INVALID_ARG;
        if (!(gd > 0.0f) || !isfinite(gd)) return W4A8_ERR_INVALID_ARG;
        rows += h_part_rows[p];
        blocks[p] = h_part_rows[p] * (K / 32);
    }
    const w4a8_status st = check_prepared_out(rows, K, mode, d_w_prepared, d_s_prepared);
    if (st != W4A8_OK) return st;
    return hip_status(launch_requant_prepared(d_nv_packed, d_nv_scale, blocks, h_part_divisor, n_parts, rows, K,
                                              (int)mode, d_w_prepared, d_s_prepared, as_stream(stream)));
}

w4a8_status w4a8_quant_bf16_to_mxfp4_prepared(const uint16_t* d_w_bf16, int64_t rows, int64_t K,
                                              w4a8_exp_mode mode, uint8_t* d_w_prepared, uint8_t* d_s_prepared,
                                              void* stream) {
    if (!d_w_bf16 || !aligned(d_w_bf16, 16)) return W4A8_ERR_INVALID_ARG;
    const w4a8_status st = check_prepared_out(rows, K, mode, d_w_prepared, d_s_prepared);
    if (st != W4A8_OK) return st;
    return hip_status(launch_quant_bf16_prepared(d_w_bf16, rows, K, (int)mode, d_w_prepared, d_s_prepared,
                                                 as_stream(stream)));
}

w4a8_status w4a8_quant_fp8ch_to_mxfp4_prepared(const uint8_t* d_w_e4m3, const float* d_row_scale, int64_t rows,
                                               int64_t K, w4a8_exp_mode mode, uint8_t* d_w_prepared,
                                               uint8_t* d_s_prepared, void* stream) {
    if (!d_w_e4m3 || !d_row_scale || !aligned(d_w_e4m3, 16) || !aligned(d_row_scale, 4))
        return W4A8_ERR_INVALID_ARG;
    const w4a8_status st = check_prepared_out(rows, K, mode, d_w_prepared, d_s_prepared);
    if (st != W4A8_OK) return st;
    if (rows * (K / 32) >= ((int64_t)1 << 32)) return W4A8_ERR_UNSUPPORTED_SHAPE;   // 32-bit block index
    return hip_status(launch_quant_fp8ch_prepared(d_w_e4m3, d_row_scale, rows, K, (int)mode, d_w_prepared,
                                                  d_s_prepared, as_stream(stream)));
}

w4a8_status w4a8_quant_act_fp8_per_token(const uint16_t* d_x_bf16, int64_t M, int64_t K,
                                         int64_t ldx, uint8_t* d_x_fp8, float* d_x_scale,
                                         void* stream) {
    if (!d_x_bf16 || !d_x_fp8 || !d_x_scale) return W4A8_ERR_INVALID_ARG;
    if (M < 1 || K < 1 || M > kMaxDim || K > kMaxDim || ldx > kMaxDim) return W4A8_ERR_INVALID_ARG;
    if (ldx < K) return W4A8_ERR_UNSUPPORTED_SHAPE;
    if (!aligned(d_x_bf16, 2) || !aligned(d_x_scale, 4)) return W4A8_ERR_INVALID_ARG;
    return hip_status(launch_act_quant(d_x_bf16, M, K, ldx, d_x_fp8, d_x_scale, as_stream(stream)));
}

// The plain-layout GEMMs above the decode band (MXFP4 [N, K/2] and the
// transposed int4 [N, K/8]; K a multiple of 128, in the tile kernel's range)
// repack the weight into fragment order inside the workspace, then run the
// tile kernel of the prepared weights.  Workspace: [split-K counters of the
// decode band, left untouched | repacked codes | repacked scales | the tile
// kernel's own workspace].
struct PlainRepack {
    size_t w_off, s_off, t_off, bytes;
};
static bool plain_repack_route(int64_t M, int64_t K) {
    return M > kDecodeMaxM && K % 128 == 0 && K <= kPreparedTiledMaxK;
}
// the linear at 17 <= M <= 64 on a wide MXFP4 layer: the codes also step-major
// ([K/128][M][128]) in the workspace, after the decode band's split-K counters
static size_t linear_sm_offset(int64_t N) { return (ws_counter_bytes((N + 15) / 16) + 255) / 256 * 256; }
static size_t linear_sm_bytes(int64_t M, int64_t N, int64_t K) {
    return linear_sm_offset(N) + (size_t)((M * K + 255) / 256 * 256);
}

static PlainRepack plain_repack_layout(int64_t N, int64_t K, size_t tiled_bytes, bool int4) {
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    size_t wb = 0, sb = 0;
    if (int4) prepared_i4_sizes(N, K, &wb, &sb);
    else prepared_sizes(N, K, &wb, &sb);
    PlainRepack r{};
    r.w_off = up(ws_counter_bytes((N + 15) / 16));
    r.s_off = r.w_off + up(wb);
    r.t_off = r.s_off + up(sb);
    r.bytes = r.t_off + tiled_bytes;
    return r;
}

size_t w4a8_gemm_workspace_bytes(int64_t M_max, int64_t N, int64_t K, w4a8_weight_kind kind) {
    if (M_max < 1 || N < 1 || K < 32 || M_max > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
    if (kind == W4A8_WEIGHT_MXFP4 && K % 32 != 0) return 0;
    if (kind == W4A8_WEIGHT_INT4G128 && (K % 128 != 0 || N % 8 != 0)) return 0;
    if (kind == W4A8_WEIGHT_MXFP4_PREPARED && K % 128 != 0) return 0;
    if (kind == W4A8_WEIGHT_INT4G128_PREPARED && (K % 128 != 0 || N % 8 != 0)) return 0;
    if (kind == W4A8_W4A4_PREPARED && K % 128 != 0) return 0;
    if (kind == W4A8_WEIGHT_INT4G128_ZP_PREPARED && (K % 128 != 0 || N % 8 != 0)) return 0;
    if (kind == W4A8_WEIGHT_INT5G128_PREPARED && K % 128 != 0) return 0;
    if (kind != W4A8_WEIGHT_MXFP4 && kind != W4A8_WEIGHT_INT4G128 && kind != W4A8_WEIGHT_MXFP4_PREPARED &&
        kind != W4A8_WEIGHT_INT4G128_PREPARED && kind != W4A8_W4A4_PREPARED &&
        kind != W4A8_WEIGHT_INT4G128_ZP_PREPARED && kind != W4A8_WEIGHT_INT5G128_PREPARED)
        return 0;
    size_t need = 0;
    auto keep = [&](size_t b) { if (b > need) need = b; };
    if (kind != W4A8_WEIGHT_MXFP4 && kind != W4A8_WEIGHT_INT4G128) {
        // fragment-order weights: the workspace a call of m rows takes, by the
        // route and shape that call gets
        auto at = [&](int64_t m) -> size_t {
            if (kind == W4A8_WEIGHT_INT5G128_PREPARED) {
                if (m > 8 && spread_fits(m, N, K)) return 0;
                if (m <= kPreparedDecodeMaxM) return plan_workspace_bytes(plan_prepared(m, N, K, 0, 0, false, true), m, N);
                return i5_tiled_fits(m, K) ? i5_tiled_workspace_bytes(m, N, K) : 0;
            }
            if (kind == W4A8_W4A4_PREPARED) return K <= kPreparedTiledMaxK ? w4a4_workspace_bytes(m, N, K) : 0;
            // the zero-point form takes the int4 kernels' routes and shapes
            const bool int4 = kind != W4A8_WEIGHT_MXFP4_PREPARED;
            const PreparedRoute r = prepared_route(m, N, K, int4);
            if (r == PreparedRoute::Decode) return plan_workspace_bytes(plan_prepared(m, N, K, 0, 0, false, int4), m, N);
            // the linear's step-major copy of the codes (more than one activation tile)
            if (r == PreparedRoute::Spread) return m > 16 && !int4 ? linear_sm_bytes(m, N, K) : 0;
            if (K > kPreparedTiledMaxK) return 0;
            if (r == PreparedRoute::DTile) return dtile_workspace_bytes(plan_dtile_route(m, N, K), m, N);
            return tiled_workspace_bytes(m, N, K, int4);
        };
        // Every M up to 64 (the decode band, whose plans change at any M).
        // Above, every tile kernel's shape (64-, 128- or 256-row tiles, the K
        // split) is constant between consecutive multiples of 64 and its split
        // workspace grows with M there, so the multiples of 64 and M_max itself
        // cover every call.  No rule splits K once even 256 x 256 tiles number
        // 1024 or more (the fewest a call of m rows can have), so the scan stops
        // there.
        for (int64_t m = 1; m <= M_max && m <= kDecodeMaxM; ++m) keep(at(m));
        const int64_t tiles_n = (N + 255) / 256;
        for (int64_t m = 2 * kDecodeMaxM; m < M_max; m += kDecodeMaxM) {
            keep(at(m));
            if ((m / 256) * tiles_n >= 1024) break;
        }
        keep(at(M_max));
        return need;
    }
    const int64_t top = M_max < kDecodeMaxM ? M_max : kDecodeMaxM;
    for (int64_t m = 1; m <= top; ++m) {
        const GemmPlan p = kind == W4A8_WEIGHT_MXFP4 ? plan_mxfp4(m, N, K) : plan_int4(m, N, K);
        const size_t b = plan_workspace_bytes(p, m, N);
        if (b > need) need = b;
    }
    if (plain_repack_route(M_max, K)) {
        // the repack and the largest tile-kernel workspace of the calls above
        // the decode band (scanned as for the prepared weights)
        const bool int4 = kind == W4A8_WEIGHT_INT4G128;
        size_t tiled = 0;
        const int64_t tiles_n = (N + 255) / 256;
        for (int64_t m = 2 * kDecodeMaxM; m < M_max; m += kDecodeMaxM) {
            const size_t b = tiled_workspace_bytes(m, N, K, int4);
            if (b > tiled) tiled = b;
            if ((m / 256) * tiles_n >= 1024) break;
        }
        const size_t b = tiled_workspace_bytes(M_max, N, K, int4);
        if (b > tiled) tiled = b;
        keep(plain_repack_layout(N, K, tiled, int4).bytes);
    }
    return need;
}

w4a8_status w4a8_workspace_init(void* d_ws, size_t bytes, void* stream) {
    if (!d_ws) return W4A8_ERR_INVALID_ARG;
    if (!aligned(d_ws, 256)) return W4A8_ERR_WORKSPACE;
    return hip_status(launch_fill_zero_u32(reinterpret_cast<uint32_t*>(d_ws), (int64_t)(bytes / 4),
                                           as_stream(stream)));
}

w4a8_status w4a8_mxfp4_gemm(const uint8_t* d_x_fp8, const float* d_x_scale,
                            const uint8_t* d_w_packed, const uint8_t* d_w_e8m0, uint16_t* d_out,
                            int64_t M, int64_t N, int64_t K, void* d_ws, size_t ws_bytes,
                            void* stream) {
    w4a8_status st = check_gemm_common(d_x_fp8, d_x_scale, d_w_packed, d_out, M, N, K);
    if (st != W4A8_OK) return st;
    if (!d_w_e8m0 || !aligned(d_w_e8m0, 4)) return W4A8_ERR_INVALID_ARG;
    if (K % 32 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    // wide layers at decode M: the spread tiles read this layout directly (no workspace)
    if (spread_plain_fits(M, N, K) && aligned(d_w_e8m0, 16))
        return hip_status(launch_spread(plan_spread(M, N, K, 0, -1), d_x_fp8, d_x_scale, d_w_packed, d_w_e8m0, d_out,
                                        M, N, K, as_stream(stream), true));
    // above the decode band: repack into fragment order in the workspace, then the tile kernel
    if (plain_repack_route(M, K)) {
        const PlainRepack r = plain_repack_layout(N, K, tiled_workspace_bytes(M, N, K, false), false);
        st = check_workspace(r.bytes, d_ws, ws_bytes);
        if (st != W4A8_OK) return st;
        uint8_t* ws = reinterpret_cast<uint8_t*>(d_ws);
        hipError_t e = launch_prepare(d_w_packed, d_w_e8m0, N, K, ws + r.w_off, ws + r.s_off, as_stream(stream));
        if (e != hipSuccess) return hip_status(e);
        return hip_status(launch_prepared_tiled(d_x_fp8, d_x_scale, ws + r.w_off, ws + r.s_off, d_out, M, N, K,
                                                ws + r.t_off, as_stream(stream), false, false, 0));
    }
    const GemmPlan p = plan_mxfp4(M, N, K);
    st = check_workspace(plan_workspace_bytes(p, M, N), d_ws, ws_bytes);
    if (st != W4A8_OK) return st;
    return hip_status(launch_mxfp4_gemm(p, d_x_fp8, d_x_scale, d_w_packed, d_w_e8m0, d_out, M, N, K,
                                        d_ws, as_stream(stream)));
}

w4a8_status w4a8_mxfp4_prepared_bytes(int64_t N, int64_t K, size_t* h_w_bytes, size_t* h_s_bytes) {
    if (!h_w_bytes || !h_s_bytes) return W4A8_ERR_INVALID_ARG;
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return W4A8_ERR_INVALID_ARG;
    if (K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    prepared_sizes(N, K, h_w_bytes, h_s_bytes);
    return W4A8_OK;
}

w4a8_status w4a8_mxfp4_prepare(const uint8_t* d_w_packed, const uint8_t* d_w_e8m0, int64_t N,
                               int64_t K, uint8_t* d_w_prepared, uint8_t* d_s_prepared,
                               void* stream) {
    if (!d_w_packed || !d_w_e8m0 || !d_w_prepared || !d_s_prepared) return W4A8_ERR_INVALID_ARG;
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return W4A8_ERR_INVALID_ARG;
    if (K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    if (!aligned(d_w_packed, 16) || !aligned(d_w_prepared, 16) || !aligned(d_s_prepared, 4))
        return W4A8_ERR_INVALID_ARG;
    return hip_status(launch_prepare(d_w_packed, d_w_e8m0, N, K, d_w_prepared, d_s_prepared,
                                     as_stream(stream)));
}

// GEMM on fragment-order weights (MXFP4, int4, int4 with zero points):
// kernel by prepared_route
static w4a8_status gemm_prepared(const uint8_t* d_x_fp8, const float* d_x_scale, const uint8_t* d_w,
                                 const uint8_t* d_s, uint16_t* d_out, int64_t M, int64_t N, int64_t K,
                                 void* d_ws, size_t ws_bytes, void* stream, bool int4, bool zp = false) {
    w4a8_status st = check_gemm_common(d_x_fp8, d_x_scale, d_w, d_out, M, N, K);
    if (st != W4A8_OK) return st;
    if (!d_s || !aligned(d_s, int4 ? 16 : 4)) return W4A8_ERR_INVALID_ARG;
    if (K % 128 != 0 || (int4 && N % 8 != 0)) return W4A8_ERR_UNSUPPORTED_SHAPE;
    // the tiled kernel addresses activations with 32-bit offsets
    const PreparedRoute route = prepared_route(M, N, K, int4);
    if (route != PreparedRoute::Decode && route != PreparedRoute::Spread && K > kPreparedTiledMaxK)
        return W4A8_ERR_UNSUPPORTED_SHAPE;
    switch (route) {
    case PreparedRoute::Spread:
        if (int4)
            return hip_status(launch_spread_i4(d_x_fp8, d_x_scale, d_w, d_s, d_out, M, N, K, as_stream(stream),
                                               zp ? 3 : 1, nullptr));
        return hip_status(launch_spread(plan_spread(M, N, K, 0, -1), d_x_fp8, d_x_scale, d_w, d_s, d_out, M, N, K,
                                        as_stream(stream)));
    case PreparedRoute::DTile: {
        const DtPlan p = plan_dtile_route(M, N, K);
        st = check_workspace(dtile_workspace_bytes(p, M, N), d_ws, ws_bytes);
        if (st != W4A8_OK) return st;
        return hip_status(launch_dtile(p, d_x_fp8, d_x_scale, d_w, d_s, d_out, M, N, K, d_ws, as_stream(stream)));
    }
    case PreparedRoute::Tiled:
        st = check_workspace(tiled_workspace_bytes(M, N, K, int4), d_ws, ws_bytes);
        if (st != W4A8_OK) return st;
        return hip_status(launch_prepared_tiled(d_x_fp8, d_x_scale, d_w, d_s, d_out, M, N, K, d_ws,
                                                as_stream(stream), int4, zp));
    default: {
        const GemmPlan p = plan_prepared(M, N, K, 0, 0, false, int4);
        st = check_workspace(plan_workspace_bytes(p, M, N), d_ws, ws_bytes);
        if (st != W4A8_OK) return st;
        return hip_status(launch_prepared_decode(p, d_x_fp8, d_x_scale, d_w, d_s, d_out, M, N, K, d_ws,
                                                 as_stream(stream), int4, zp));
    }
    }
}

// ---- GEMM on prepared MXFP4 weights with no caller workspace ----
//
// The split-K partials of w4a8_mxfp4_gemm_prepared_noalloc live in this
// file-scope device array: one copy on every GPU the library runs on, held
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: host code only ever uses the device address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch).  The
// array starts zeroed (static device storage), as the split-K arrival
// counters at its start must be; every call leaves them at zero again, and no
// kernel reads a partial before its split has written it, so the array needs
// no clearing between calls.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up on the
// first call per device (with that device current) and kept.
hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

// the linear on bf16 activations: fused per-token quant in the decode kernel
// where the plan allows it, else the quant kernel then gemm_prepared
static w4a8_status linear_prepared(const uint16_t* d_x_bf16, int64_t ldx, const uint8_t* d_w, const uint8_t* d_s,
                                   uint16_t* d_out, int64_t M, int64_t N, int64_t K, uint8_t* d_x_fp8,
                                   float* d_x_scale, void* d_ws, size_t ws_bytes, void* stream, bool int4) {
    if (!d_x_bf16 || !aligned(d_x_bf16, 2)) return W4A8_ERR_INVALID_ARG;
    if (ldx < K || ldx > kMaxDim) return ldx < K ? W4A8_ERR_UNSUPPORTED_SHAPE : W4A8_ERR_INVALID_ARG;
    w4a8_status st = check_gemm_common(d_x_fp8, d_x_scale, d_w, d_out, M, N, K);
    if (st != W4A8_OK) return st;
    if (!d_s || !aligned(d_s, int4 ? 16 : 4)) return W4A8_ERR_INVALID_ARG;
    if (K % 128 != 0 || (int4 && N % 8 != 0)) return W4A8_ERR_UNSUPPORTED_SHAPE;
    GemmPlan p{};
    const bool vec = aligned(d_x_bf16, 16) && ldx % 8 == 0;
    // the quantization fused into the split-K decode kernel where its plan
    // allows, also for one row on wide layers whose GEMM alone takes the spread
    // tiles (gate_up M = 1: 19.1 us fused against 20.4 us for quant kernel + spread)
    const PreparedRoute route = prepared_route(M, N, K, int4);
    // one token on a wide layer: the quantization fused into the spread tiles
    if (!int4 && vec && route == PreparedRoute::Spread && spread_fq_fits(M, N, K))
        return hip_status(launch_spread_fq(d_x_bf16, d_w, d_s, d_out, d_x_fp8, d_x_scale, N, K, as_stream(stream)));
    if (vec && (route == PreparedRoute::Decode || (route == PreparedRoute::Spread && M == 1)) &&
        plan_prepared_fused(M, N, K, int4, &p))
        return hip_status(launch_prepared_linear_fused(p, d_x_bf16, ldx, d_w, d_s, d_out, M, N, K, d_x_fp8,
                                                       d_x_scale, as_stream(stream), int4));
    // more than one activation tile on a wide layer: the quant kernel also
    // writes the codes step-major into the workspace (a step's rows contiguous),
    // which the spread tiles stage from (gate_up M = 32 / 64: 18.4 / 21.3 us on
    // the row-major codes, 17.8 / 20.4 step-major; no gain at M <= 16, where
    // the staged rows are 16 lines a step); without room, the codes as written
    if (!int4 && route == PreparedRoute::Spread && M > 16 && act_quant_sm_fits(d_x_bf16, M, K, ldx, d_x_fp8) &&
        d_ws && aligned(d_ws, 256) && ws_bytes >= linear_sm_bytes(M, N, K)) {
        uint8_t* x8s = static_cast<uint8_t*>(d_ws) + linear_sm_offset(N);
        st = hip_status(launch_act_quant_sm(d_x_bf16, M, K, ldx, d_x_fp8, d_x_scale, x8s, as_stream(stream)));
        if (st != W4A8_OK) return st;
        return hip_status(launch_spread(plan_spread(M, N, K, 0, -1), x8s, d_x_scale, d_w, d_s, d_out, M, N, K,
                                        as_stream(stream), false, true));
    }
    st = hip_status(launch_act_quant(d_x_bf16, M, K, ldx, d_x_fp8, d_x_scale, as_stream(stream)));
    if (st != W4A8_OK) return st;
    return gemm_prepared(d_x_fp8, d_x_scale, d_w, d_s, d_out, M, N, K, d_ws, ws_bytes, stream, int4);
}

w4a8_status w4a8_mxfp4_gemm_prepared_noalloc(const uint8_t* d_x_fp8, const float* d_x_scale,
                                             const uint8_t* d_w_prepared, const uint8_t* d_s_prepared,
                                             uint16_t* d_out, int64_t M, int64_t N, int64_t K, void* stream) {
    w4a8_status st = check_gemm_common(d_x_fp8, d_x_scale, d_w_prepared, d_out, M, N, K);
    if (st != W4A8_OK) return st;
    void* ws = nullptr;
    if (noalloc_scratch(&ws) != hipSuccess) return W4A8_ERR_HIP;
    // a call whose split-K partials exceed the array fails in gemm_prepared's
    // workspace check (W4A8_ERR_WORKSPACE) before anything is enqueued
    return gemm_prepared(d_x_fp8, d_x_scale, d_w_prepared, d_s_prepared, d_out, M, N, K, ws,
                         kNoAllocScratchBytes, stream, false);
}

size_t w4a8_mxfp4_gemm_prepared_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

w4a8_status w4a8_mxfp4_linear_prepared(const uint16_t* d_x_bf16, int64_t ldx, const uint8_t* d_w_prepared,
                                       const uint8_t* d_s_prepared, uint16_t* d_out, int64_t M, int64_t N,
                                       int64_t K, uint8_t* d_x_fp8, float* d_x_scale, void* d_ws,
                                       size_t ws_bytes, void* stream) {
    return linear_prepared(d_x_bf16, ldx, d_w_prepared, d_s_prepared, d_out, M, N, K, d_x_fp8, d_x_scale, d_ws,
                           ws_bytes, stream, false);
}

w4a8_status w4a8_int4g128_linear_prepared(const uint16_t* d_x_bf16, int64_t ldx, const uint8_t* d_w_prepared,
                                          const uint8_t* d_s_prepared, uint16_t* d_out, int64_t M, int64_t N,
                                          int64_t K, uint8_t* d_x_fp8, float* d_x_scale, void* d_ws,
                                          size_t ws_bytes, void* stream) {
    return linear_prepared(d_x_bf16, ldx, d_w_prepared, d_s_prepared, d_out, M, N, K, d_x_fp8, d_x_scale, d_ws,
                           ws_bytes, stream, true);
}

w4a8_status w4a8_mxfp4_gemm_prepared(const uint8_t* d_x_fp8, const float* d_x_scale,
                                     const uint8_t* d_w_prepared, const uint8_t* d_s_prepared,
                                     uint16_t* d_out, int64_t M, int64_t N, int64_t K, void* d_ws,
                                     size_t ws_bytes, void* stream) {
    return gemm_prepared(d_x_fp8, d_x_scale, d_w_prepared, d_s_prepared, d_out, M, N, K, d_ws, ws_bytes,
                         stream, false);
}

w4a8_status w4a8_w4a4_gemm_prepared(const uint8_t* d_x_fp4, const uint8_t* d_x_e8m0,
                                    const uint8_t* d_w_prepared, const uint8_t* d_s_prepared, uint16_t* d_out,
                                    int64_t M, int64_t N, int64_t K, void* d_ws, size_t ws_bytes, void* stream) {
    w4a8_status st = check_gemm_common(d_x_fp4, d_x_e8m0, d_w_prepared, d_out, M, N, K);
    if (st != W4A8_OK) return st;
    if (!d_s_prepared || !aligned(d_s_prepared, 4) || !aligned(d_x_fp4, 16) || !aligned(d_x_e8m0, 4))
        return W4A8_ERR_INVALID_ARG;
    if (K % 128 != 0 || K > kPreparedTiledMaxK) return W4A8_ERR_UNSUPPORTED_SHAPE;
    st = check_workspace(w4a4_workspace_bytes(M, N, K), d_ws, ws_bytes);
    if (st != W4A8_OK) return st;
    return hip_status(launch_prepared_w4a4(d_x_fp4, d_x_e8m0, d_w_prepared, d_s_prepared, d_out, M, N, K, d_ws,
                                           as_stream(stream)));
}

w4a8_status w4a8_int4g128_prepared_bytes(int64_t N, int64_t K, size_t* h_w_bytes, size_t* h_s_bytes) {
    if (!h_w_bytes || !h_s_bytes) return W4A8_ERR_INVALID_ARG;
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return W4A8_ERR_INVALID_ARG;
    if (N % 8 != 0 || K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    prepared_i4_sizes(N, K, h_w_bytes, h_s_bytes);
    return W4A8_OK;
}

w4a8_status w4a8_int4g128_prepare_fragments(const int32_t* d_qweight_kn, const int32_t* d_qzeros,
                                            const uint16_t* d_scales_f16, int64_t N, int64_t K,
                                            uint8_t* d_w_prepared, uint8_t* d_s_prepared, void* stream) {
    if (!d_qweight_kn || !d_qzeros || !d_scales_f16 || !d_w_prepared || !d_s_prepared)
        return W4A8_ERR_INVALID_ARG;
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return W4A8_ERR_INVALID_ARG;
    if (N % 8 != 0 || K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    if (!aligned(d_qweight_kn, 4) || !aligned(d_qzeros, 4) || !aligned(d_scales_f16, 2) ||
        !aligned(d_w_prepared, 16) || !aligned(d_s_prepared, 16))
        return W4A8_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    // the first prepared word serves as the mismatch counter before the repack
    uint32_t* counter = reinterpret_cast<uint32_t*>(d_w_prepared);
    if (launch_fill_zero_u32(counter, 1, s) != hipSuccess) return W4A8_ERR_HIP;
    if (launch_int4_check_transpose(nullptr, d_qzeros, N, K, nullptr, counter, s) != hipSuccess)
        return W4A8_ERR_HIP;
    uint32_t bad = 0;
    if (hipMemcpyAsync(&bad, counter, sizeof(bad), hipMemcpyDeviceToHost, s) != hipSuccess)
        return W4A8_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return W4A8_ERR_HIP;
    if (bad) return W4A8_ERR_ASYMMETRIC;
    return hip_status(launch_prepare_i4(d_qweight_kn, d_scales_f16, N, K, d_w_prepared, d_s_prepared, s));
}

w4a8_status w4a8_int4g128_gemm_prepared(const uint8_t* d_x_fp8, const float* d_x_scale,
                                        const uint8_t* d_w_prepared, const uint8_t* d_s_prepared,
                                        uint16_t* d_out, int64_t M, int64_t N, int64_t K, void* d_ws,
                                        size_t ws_bytes, void* stream) {
    return gemm_prepared(d_x_fp8, d_x_scale, d_w_prepared, d_s_prepared, d_out, M, N, K, d_ws, ws_bytes,
                         stream, true);
}

w4a8_status w4a8_int4g128_zp_prepared_bytes(int64_t N, int64_t K, size_t* h_w_bytes, size_t* h_s_bytes) {
    if (!h_w_bytes || !h_s_bytes) return W4A8_ERR_INVALID_ARG;
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return W4A8_ERR_INVALID_ARG;
    if (N % 8 != 0 || K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    prepared_i4z_sizes(N, K, h_w_bytes, h_s_bytes);
    return W4A8_OK;
}

w4a8_status w4a8_int4g128_zp_prepare_fragments(const int32_t* d_qweight_kn, const int32_t* d_qzeros,
                                               const uint16_t* d_scales_f16, int64_t N, int64_t K,
                                               uint8_t* d_w_prepared, uint8_t* d_s_prepared, void* stream) {
    if (!d_qweight_kn || !d_qzeros || !d_scales_f16 || !d_w_prepared || !d_s_prepared)
        return W4A8_ERR_INVALID_ARG;
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return W4A8_ERR_INVALID_ARG;
    if (N % 8 != 0 || K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    if (!aligned(d_qweight_kn, 4) || !aligned(d_qzeros, 4) || !aligned(d_scales_f16, 2) ||
        !aligned(d_w_prepared, 16) || !aligned(d_s_prepared, 16))
        return W4A8_ERR_INVALID_ARG;
    return hip_status(launch_prepare_i4z(d_qweight_kn, d_qzeros, d_scales_f16, N, K, d_w_prepared, d_s_prepared,
                                         as_stream(stream)));
}

w4a8_status w4a8_int4g128_zp_gemm_prepared(const uint8_t* d_x_fp8, const float* d_x_scale,
                                           const uint8_t* d_w_prepared, const uint8_t* d_s_prepared,
                                           uint16_t* d_out, int64_t M, int64_t N, int64_t K, void* d_ws,
                                           size_t ws_bytes, void* stream) {
    if (d_s_prepared && !aligned(d_s_prepared, 16)) return W4A8_ERR_INVALID_ARG;
    return gemm_prepared(d_x_fp8, d_x_scale, d_w_prepared, d_s_prepared, d_out, M, N, K, d_ws, ws_bytes,
                         stream, true, true);
}

w4a8_status w4a8_int5g128_prepared_bytes(int64_t N, int64_t K, size_t* h_w_bytes, size_t* h_w5_bytes,
                                         size_t* h_s_bytes) {
    if (!h_w_bytes || !h_w5_bytes || !h_s_bytes) return W4A8_ERR_INVALID_ARG;
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return W4A8_ERR_INVALID_ARG;
    if (K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    prepared_i5_sizes(N, K, h_w_bytes, h_w5_bytes, h_s_bytes);
    return W4A8_OK;
}

w4a8_status w4a8_int5g128_prepare_fragments(const int32_t* d_qweight_kn, const int32_t* d_qweight_hi,
                                            const uint8_t* d_qzeros, const uint16_t* d_scales_f16, int64_t N,
                                            int64_t K, uint8_t* d_w_prepared, uint8_t* d_w5_prepared,
                                            uint8_t* d_s_prepared, void* stream) {
    if (!d_qweight_kn || !d_qweight_hi || !d_qzeros || !d_scales_f16 || !d_w_prepared || !d_w5_prepared ||
        !d_s_prepared)
        return W4A8_ERR_INVALID_ARG;
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return W4A8_ERR_INVALID_ARG;
    if (K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    if (!aligned(d_qweight_kn, 4) || !aligned(d_qweight_hi, 4) || !aligned(d_scales_f16, 2) ||
        !aligned(d_w_prepared, 16) || !aligned(d_w5_prepared, 16) || !aligned(d_s_prepared, 16))
        return W4A8_ERR_INVALID_ARG;
    return hip_status(launch_prepare_i5(d_qweight_kn, d_qweight_hi, d_qzeros, d_scales_f16, N, K, d_w_prepared,
                                        d_w5_prepared, d_s_prepared, as_stream(stream)));
}

w4a8_status w4a8_int5g128_gemm_prepared(const uint8_t* d_x_fp8, const float* d_x_scale,
                                        const uint8_t* d_w_prepared, const uint8_t* d_w5_prepared,
                                        const uint8_t* d_s_prepared, uint16_t* d_out, int64_t M, int64_t N,
                                        int64_t K, void* d_ws, size_t ws_bytes, void* stream) {
    w4a8_status st = check_gemm_common(d_x_fp8, d_x_scale, d_w_prepared, d_out, M, N, K);
    if (st != W4A8_OK) return st;
    if (!d_w5_prepared || !d_s_prepared || !aligned(d_w5_prepared, 16) || !aligned(d_s_prepared, 16))
        return W4A8_ERR_INVALID_ARG;
    if (K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    hipStream_t s = as_stream(stream);
    // wide layers from 9 to 64 rows: the spread tiles (no workspace)
    if (M > 8 && spread_fits(M, N, K))
        return hip_status(launch_spread_i4(d_x_fp8, d_x_scale, d_w_prepared, d_s_prepared, d_out, M, N, K, s, 4,
                                           d_w5_prepared));
    if (M <= kPreparedDecodeMaxM) {
        // the split-K decode kernel
        st = check_workspace(plan_workspace_bytes(plan_prepared(M, N, K, 0, 0, false, true), M, N), d_ws, ws_bytes);
        if (st != W4A8_OK) return st;
        return hip_status(launch_prepared_decode_i5(d_x_fp8, d_x_scale, d_w_prepared, d_w5_prepared, d_s_prepared,
                                                    d_out, M, N, K, d_ws, s));
    }
    // the tile kernel (its activation-sum pre-pass writes the workspace)
    if (!i5_tiled_fits(M, K)) return W4A8_ERR_UNSUPPORTED_SHAPE;
    st = check_workspace(i5_tiled_workspace_bytes(M, N, K), d_ws, ws_bytes);
    if (st != W4A8_OK) return st;
    return hip_status(launch_prepared_tiled_i5(d_x_fp8, d_x_scale, d_w_prepared, d_w5_prepared, d_s_prepared, d_out,
                                               M, N, K, d_ws, s));
}

w4a8_status w4a8_int4g128_prepare(const int32_t* d_qweight_kn, const int32_t* d_qzeros, int64_t N,
                                  int64_t K, int32_t* d_qweight_nk, void* stream) {
    if (!d_qweight_kn || !d_qzeros || !d_qweight_nk) return W4A8_ERR_INVALID_ARG;
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return W4A8_ERR_INVALID_ARG;
    if (N % 8 != 0 || K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    if (!aligned(d_qweight_kn, 4) || !aligned(d_qzeros, 4) || !aligned(d_qweight_nk, 4))
        return W4A8_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    // the first output word serves as the mismatch counter before the transpose
    uint32_t* counter = reinterpret_cast<uint32_t*>(d_qweight_nk);
    if (launch_fill_zero_u32(counter, 1, s) != hipSuccess) return W4A8_ERR_HIP;
    if (launch_int4_check_transpose(nullptr, d_qzeros, N, K, nullptr, counter, s) != hipSuccess)
        return W4A8_ERR_HIP;
    uint32_t bad = 0;
    if (hipMemcpyAsync(&bad, counter, sizeof(bad), hipMemcpyDeviceToHost, s) != hipSuccess)
        return W4A8_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return W4A8_ERR_HIP;
    if (bad) return W4A8_ERR_ASYMMETRIC;
    return hip_status(launch_int4_check_transpose(d_qweight_kn, nullptr, N, K, d_qweight_nk, nullptr, s));
}

w4a8_status w4a8_int4g128_gemm(const uint8_t* d_x_fp8, const float* d_x_scale,
                               const int32_t* d_qweight_nk, const uint16_t* d_scales_f16,
                               uint16_t* d_out, int64_t M, int64_t N, int64_t K, void* d_ws,
                               size_t ws_bytes, void* stream) {
    w4a8_status st = check_gemm_common(d_x_fp8, d_x_scale, d_qweight_nk, d_out, M, N, K);
    if (st != W4A8_OK) return st;
    if (!d_scales_f16 || !aligned(d_scales_f16, 8)) return W4A8_ERR_INVALID_ARG;
    if (N % 8 != 0 || K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    // above the decode band: repack into fragment order in the workspace, then the tile kernel
    if (plain_repack_route(M, K)) {
        const PlainRepack r = plain_repack_layout(N, K, tiled_workspace_bytes(M, N, K, true), true);
        st = check_workspace(r.bytes, d_ws, ws_bytes);
        if (st != W4A8_OK) return st;
        uint8_t* ws = reinterpret_cast<uint8_t*>(d_ws);
        hipError_t e = launch_prepare_i4_nk(d_qweight_nk, d_scales_f16, N, K, ws + r.w_off, ws + r.s_off,
                                            as_stream(stream));
        if (e != hipSuccess) return hip_status(e);
        return hip_status(launch_prepared_tiled(d_x_fp8, d_x_scale, ws + r.w_off, ws + r.s_off, d_out, M, N, K,
                                                ws + r.t_off, as_stream(stream), true, false, 0));
    }
    const GemmPlan p = plan_int4(M, N, K);
    st = check_workspace(plan_workspace_bytes(p, M, N), d_ws, ws_bytes);
    if (st != W4A8_OK) return st;
    return hip_status(launch_int4_gemm(p, d_x_fp8, d_x_scale, d_qweight_nk, d_scales_f16, d_out, M,
                                       N, K, d_ws, as_stream(stream)));
}

// ---- decode band with an explicit plan (tile-size sweeps) ----

size_t w4a8_decode_plan_workspace_bytes(int64_t M, int64_t N, int64_t K, int rt, int u, int ks) {
    if (M < 1 || M > kDecodeMaxM || N < 1 || K < 32 || N > kMaxDim || K > kMaxDim) return 0;
    if (rt == 0) {   // prepared weights: u = ring depth
        if (M > kPreparedDecodeMaxM || K % 128 != 0 || u < 2 || u > 4 || ks < 1) return 0;
        return plan_workspace_bytes(plan_prepared(M, N, K, ks, u, false, false), M, N);
    }
    if (rt > 100) {   // prepared weights, split-K decode kernel: rt - 100 tiles x ks K parts per workgroup
        if (u < 2 || u > 4 || ks < 1 || (rt - 100) * ks > 16 || M > kPreparedDecodeMaxM || K % 128 != 0) return 0;
        return plan_workspace_bytes(plan_prepared_explicit(M, N, K, rt - 100, ks, u), M, N);
    }
    if (rt == -200) return 0;   // prepared weights, spread tiles (ring depth ks, 0: default): no workspace
    if (rt == -100) {   // prepared weights, the tiled kernel with K split in ks
        if (K % 128 != 0 || ks < 1) return 0;
        return tiled_workspace_bytes(M, N, K, false, ks);
    }
    if (rt < 0) {    // prepared weights, register-streamed tiles: -rt tiles per wave
        if (K % 128 != 0 || (rt != -1 && rt != -2 && rt != -4) || (u != 4 && u != 8 && u != 16) || ks < 1)
            return 0;
        return dtile_workspace_bytes(plan_dtile(M, N, K, -rt, u, ks), M, N);
    }
    if ((rt != 1 && rt != 2 && rt != 4) || (u != 1 && u != 2 && u != 4) || ks < 1) return 0;
    return plan_workspace_bytes(make_decode_plan(M, N, K, rt, u, ks), M, N);
}

w4a8_status w4a8_decode_with_plan(w4a8_weight_kind kind, const uint8_t* d_x_fp8,
                                  const float* d_x_scale, const void* d_w, const void* d_w_scale,
                                  uint16_t* d_out, int64_t M, int64_t N, int64_t K, int rt, int u,
                                  int ks, void* d_ws, size_t ws_bytes, void* stream) {
    w4a8_status st = check_gemm_common(d_x_fp8, d_x_scale, d_w, d_out, M, N, K);
    if (st != W4A8_OK) return st;
    if (kind == W4A8_WEIGHT_MXFP4_PREPARED && rt == -100) {
        if (!d_w_scale || !aligned(d_w_scale, 4) || ks < 1) return W4A8_ERR_INVALID_ARG;
        if (K % 128 != 0 || K > kPreparedTiledMaxK) return W4A8_ERR_UNSUPPORTED_SHAPE;
        st = check_workspace(tiled_workspace_bytes(M, N, K, false, ks), d_ws, ws_bytes);
        if (st != W4A8_OK) return st;
        return hip_status(launch_prepared_tiled(d_x_fp8, d_x_scale, (const uint8_t*)d_w, (const uint8_t*)d_w_scale,
                                                d_out, M, N, K, d_ws, as_stream(stream), false, false, ks));
    }
    if (kind == W4A8_WEIGHT_MXFP4_PREPARED && rt == -200) {
        // ks = ring depth (0: the entry point's), plus 100 for the e8m0 dwords once per chunk
        const int depth = ks % 100, cs = ks / 100;
        if (!d_w_scale || !aligned(d_w_scale, 4) || (depth != 0 && depth != 4 && depth != 8) || cs > 1 ||
            (cs && depth != 4))
            return W4A8_ERR_INVALID_ARG;
        // the ring turns in whole trips over the padded steps
        const int64_t s_pad = 4 * ((K / 128 + 3) / 4);
        if (K % 128 != 0 || M > 64 || (depth != 0 && s_pad % depth != 0) || (cs && s_pad % 8 != 0))
            return W4A8_ERR_UNSUPPORTED_SHAPE;
        const SpPlan p = plan_spread(M, N, K, depth, cs);
        return hip_status(launch_spread(p, d_x_fp8, d_x_scale, (const uint8_t*)d_w, (const uint8_t*)d_w_scale, d_out,
                                        M, N, K, as_stream(stream)));
    }
    if (kind == W4A8_WEIGHT_MXFP4_PREPARED && rt < 0) {
        if (!d_w_scale || !aligned(d_w_scale, 4) || (rt != -1 && rt != -2 && rt != -4) ||
            (u != 4 && u != 8 && u != 16) || ks < 1)
            return W4A8_ERR_INVALID_ARG;
        if (K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
        const DtPlan p = plan_dtile(M, N, K, -rt, u, ks);
        st = check_workspace(dtile_workspace_bytes(p, M, N), d_ws, ws_bytes);
        if (st != W4A8_OK) return st;
        return hip_status(launch_dtile(p, d_x_fp8, d_x_scale, (const uint8_t*)d_w, (const uint8_t*)d_w_scale,
                                       d_out, M, N, K, d_ws, as_stream(stream)));
    }
    if (kind == W4A8_WEIGHT_MXFP4_PREPARED) {
        if (!d_w_scale || !aligned(d_w_scale, 4) || M > kPreparedDecodeMaxM || u < 2 || u > 4 || ks < 1 ||
            (rt != 0 && (rt <= 100 || (rt - 100) * ks > 16)))
            return W4A8_ERR_INVALID_ARG;
        if (K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
        const GemmPlan p = rt > 100 ? plan_prepared_explicit(M, N, K, rt - 100, ks, u)
                                    : plan_prepared(M, N, K, ks, u, false, false);
        st = check_workspace(plan_workspace_bytes(p, M, N), d_ws, ws_bytes);
        if (st != W4A8_OK) return st;
        return hip_status(launch_prepared_decode(p, d_x_fp8, d_x_scale, (const uint8_t*)d_w,
                                                 (const uint8_t*)d_w_scale, d_out, M, N, K, d_ws,
                                                 as_stream(stream), false, false));
    }
    if (M > kDecodeMaxM || (rt != 1 && rt != 2 && rt != 4) || (u != 1 && u != 2 && u != 4) || ks < 1)
        return W4A8_ERR_INVALID_ARG;
    if (kind == W4A8_WEIGHT_MXFP4) {
        if (!d_w_scale || !aligned(d_w_scale, 4)) return W4A8_ERR_INVALID_ARG;
        if (K % 32 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    } else if (kind == W4A8_WEIGHT_INT4G128) {
        if (!d_w_scale || !aligned(d_w_scale, 8)) return W4A8_ERR_INVALID_ARG;
        if (N % 8 != 0 || K % 128 != 0) return W4A8_ERR_UNSUPPORTED_SHAPE;
    } else {
        return W4A8_ERR_INVALID_ARG;
    }
    const GemmPlan p = make_decode_plan(M, N, K, rt, u, ks);
    st = check_workspace(plan_workspace_bytes(p, M, N), d_ws, ws_bytes);
    if (st != W4A8_OK) return st;
    if (kind == W4A8_WEIGHT_MXFP4)
        return hip_status(launch_mxfp4_gemm(p, d_x_fp8, d_x_scale, (const uint8_t*)d_w,
                                            (const uint8_t*)d_w_scale, d_out, M, N, K, d_ws,
                                            as_stream(stream)));
    return hip_status(launch_int4_gemm(p, d_x_fp8, d_x_scale, (const int32_t*)d_w,
                                       (const uint16_t*)d_w_scale, d_out, M, N, K, d_ws,
                                       as_stream(stream)));
}

const char* w4a8_status_string(w4a8_status s) {
    switch (s) {
        case W4A8_OK: return "ok";
        case W4A8_ERR_INVALID_ARG: return "invalid argument";
        case W4A8_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case W4A8_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case W4A8_ERR_ASYMMETRIC: return "int4 zero points are not all 8 (asymmetric)";
        case W4A8_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* w4a8_version(void) { return "w4a8 0.1.0 gfx950"; }

}  // extern "C"
