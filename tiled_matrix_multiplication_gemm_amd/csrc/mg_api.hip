// C ABI of libmi355gemm.so: argument validation (host only, before any HIP
// call), configuration selection from the static table, and kernel launch on
// the caller's stream.  See include/mi355gemm.h for the contract.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <type_traits>
#include <stdint.h>

#include "mi355gemm.h"
#include "mg_im2col.h"
#include "mg_table.h"
#include "mg_rates.h"

namespace {

using namespace mg;

template <class C, class F>
constexpr mg_config_desc describe(int id, const char* name) {
    if constexpr (std::is_void<F>::value)
        return mg_config_desc{id, C::BM, C::BN, C::BK, C::WM, C::WN, C::STAGES, 32, 32, 16, kGroupM, 1,
                              C::LDS_BYTES, 0, 0, 0, 0, 0, name};
    else if constexpr (is_slab<F>::value)
        return mg_config_desc{id, C::BM, C::BN, C::BK, C::WM, C::WN, C::STAGES, 32, 32, 16, kGroupM, 1,
                              C::LDS_BYTES, 1, F::BK, F::STAGES, F::LDS_BYTES, F::NW, name};
    else
        return mg_config_desc{id, C::BM, C::BN, C::BK, C::WM, C::WN, C::STAGES, 32, 32, 16, kGroupM, 1,
                              C::LDS_BYTES, 1, F::BK, F::STAGES, F::LDS_BYTES, 1, name};
}

const mg_config_desc kTable[kNumConfigs] = {
    describe<Cfg0, Fast0>(0, "t256x256_w2x4_k32r5"), describe<Cfg1, Fast1>(1, "t128x128_w2x2_2cu"),
    describe<Cfg2, Fast2>(2, "t64x64_w2x2_2cu"),   describe<Cfg3, Fast3>(3, "t128x256_w2x2"),
    describe<Cfg4, Fast4>(4, "t256x128_w4x2_2cu"), describe<Cfg5, void>(5, "t128x128k32_w2x2"),
    describe<Cfg6, Fast6>(6, "t256x256_w2x2_k32r5"), describe<Cfg7, Fast7>(7, "t64x64_ksplit4"),
    describe<Cfg8, Fast8>(8, "t256x64_w4x2"),  describe<Cfg9, Fast9>(9, "t256x64_w4x1_2cu"),
};

std::atomic<int> g_forced{-1};
std::atomic<int> g_group_m{-1};  // raster overrides (mg_set_raster); -1: the table's
std::atomic<int> g_xcd{-1};
std::atomic<int> g_last{-1};
std::atomic<int> g_last_kernel{-1};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Row choice.  A workgroup's tile runs on one CU, and the tiles run in
// rounds of 256 (one per CU), so the time of a row is modelled as
// rounds * (BM * BN * K * kSecPerElemK / rate + kFixedSec), with the row's
// per-CU output rate, the seconds per output element and k, and the fixed
// time per tile fitted by the offline sweep (mg_rates.h, generated from
// profiles/table_sweep.json).  A shape the sweep timed takes the row that
// measured fastest on it (the cached top-1 of "Using Triton to optimise GEMM
// across chips", section 3.3); swept shapes are keyed by the expert count
// (grouped) and the batch count (batched products such as attention scores)
// as well.  Grouped problems count the tiles of E experts with T / E rows
// each (the host does not read the device offsets); a batched product counts
// the tiles of every entry.
double model_seconds(const rates::RowRate& r, int64_t tiles, int64_t K) {
    // each CU works through ceil(tiles / 256) tiles; a row holding `occ`
    // workgroups per CU pays the fixed time once per `occ` of them
    return (double)cdiv(tiles, 256) * (double)r.bm * r.bn * (double)K * rates::kSecPerElemK / r.rate +
           (double)cdiv(tiles, 256 * (int64_t)r.occ) * rates::kFixedSec;
}

int64_t tiles_of(const rates::RowRate& r, int64_t M, int64_t N, int64_t experts, int64_t batch) {
    if (experts > 0) return experts * cdiv(cdiv(M, experts), r.bm) * cdiv(N, r.bn);
    return cdiv(M, r.bm) * cdiv(N, r.bn) * (batch > 1 ? batch : 1);
}

int select_config(int64_t M, int64_t N, int64_t K, int64_t experts, int64_t batch = 1) {
    int forced = g_forced.load();
    if (forced >= 0) return forced;
    const int64_t b = batch > 1 ? batch : 1;
    for (const rates::Swept& sw : rates::kSwept)
        if (sw.M == M && sw.N == N && sw.K == K && sw.experts == experts && sw.batch == b) return sw.row;
    int best = rates::kRows[0].id;
    double best_t = -1.0;
    for (const rates::RowRate& r : rates::kRows) {
        const double t = model_seconds(r, tiles_of(r, M, N, experts, batch), K);
        if (best_t < 0.0 || t < best_t) {
            best_t = t;
            best = r.id;
        }
    }
    return best;
}

// Split-K runs on the rows whose fast kernel serves small and mid-size
// tiles (0, 1, 2), chosen by the same model with the tiles of every split
// counted and K / splits per tile.
bool splitk_row(int id) { return id == 0 || id == 1 || id == 2; }

double splitk_seconds(int64_t M, int64_t N, int64_t K, int64_t splits, int* row) {
    double best_t = -1.0;
    for (const rates::RowRate& r : rates::kRows) {
        if (!splitk_row(r.id)) continue;
        const double t = model_seconds(r, tiles_of(r, M, N, 0, 1) * splits, cdiv(K, splits));
        if (best_t < 0.0 || t < best_t) {
            best_t = t;
            if (row) *row = r.id;
        }
    }
    // the fp32 partials, written and read back
    if (splits > 1) best_t += 2.0 * (double)splits * (double)M * (double)N * 4.0 / rates::kPartialBytesPerSec;
    return best_t;
}

int select_config_splitk(int64_t M, int64_t N, int64_t K, int64_t splits) {
    int forced = g_forced.load();
    if (forced >= 0) return forced;
    int row = 2;
    splitk_seconds(M, N, K, splits, &row);
    return row;
}

// ---- validation --------------------------------------------------------------
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// A rows x cols matrix with row stride ld and inner stride inner.
mg_status check_matrix(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t inner, int esize = 2) {
    if (rows < 0 || cols < 0) return MG_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return MG_OK;  // no extent: never dereferenced
    if (p == nullptr) return MG_ERR_INVALID_ARG;
    if (cols > 1 && inner != 1) return MG_ERR_UNSUPPORTED_LAYOUT;
    if (rows > 1 && ld < cols) return MG_ERR_UNSUPPORTED_LAYOUT;
    if (!aligned16(p)) return MG_ERR_MISALIGNED;
    if (rows > 1 && (ld * esize) % 16 != 0) return MG_ERR_MISALIGNED;
    return MG_OK;
}

mg_status check_dtype(mg_dtype in, mg_dtype out) {
    if ((in != MG_F16 && in != MG_BF16) || in != out) return MG_ERR_UNSUPPORTED_DTYPE;
    return MG_OK;
}

#define MG_TRY(expr)                         \
    do {                                     \
        mg_status s_ = (expr);               \
        if (s_ != MG_OK) return s_;          \
    } while (0)

// ---- launch --------------------------------------------------------------------
mg_status launch(int cfg, int dt, bool epi, int mode, KArgs& a, hipStream_t s, int ta = 0, int tb = 0) {
    const mg_config_desc& d = kTable[cfg];
    // tile counts in 64 bits, checked before they are narrowed: grouped
    // launches size the grid for the worst case, one partial tile per expert
    const int64_t tn = cdiv(a.N, d.bn);
    const int64_t tm = cdiv(a.M, d.bm) + (mode == MODE_GROUPED ? a.E : 0);
    if (tn > 0x7fffffff || tm > 0x7fffffff || tm * tn > 0x7fffffff) return MG_ERR_INVALID_ARG;
    int64_t grid = tm * tn;
    if (mode == MODE_SPLITK) grid *= a.splits;
    else if (mode != MODE_GROUPED && a.batch > 1) grid *= a.batch;
    if (grid <= 0) return MG_OK;
    if (grid > 0x7fffffff) return MG_ERR_INVALID_ARG;
    a.tiles_n = (int32_t)tn;
    a.tiles_m = mode == MODE_GROUPED ? 0 : (int32_t)tm;
    a.grid = (int32_t)grid;
    const int gm = g_group_m.load(), xr = g_xcd.load();
    a.group_m = gm > 0 ? gm : d.group_m;
    a.xcd_remap = xr >= 0 ? xr : d.xcd_remap;
    mg_status st;
    switch (cfg) {
        case 0: st = launch_row0(dt, epi, mode, ta, tb, a, grid, s); break;
        case 1: st = launch_row1(dt, epi, mode, ta, tb, a, grid, s); break;
        case 2: st = launch_row2(dt, epi, mode, ta, tb, a, grid, s); break;
        case 3: st = launch_row3(dt, epi, mode, ta, tb, a, grid, s); break;
        case 4: st = launch_row4(dt, epi, mode, ta, tb, a, grid, s); break;
        case 5: st = launch_row5(dt, epi, mode, ta, tb, a, grid, s); break;
        case 6: st = launch_row6(dt, epi, mode, ta, tb, a, grid, s); break;
        case 7: st = launch_row7(dt, epi, mode, ta, tb, a, grid, s); break;
        case 8: st = launch_row8(dt, epi, mode, ta, tb, a, grid, s); break;
        case 9: st = launch_row9(dt, epi, mode, ta, tb, a, grid, s); break;
        default: return MG_ERR_BAD_CONFIG;
    }
    if (st == MG_OK && !a.dry) g_last.store(cfg);
    return st;
}

// fp32 tile by how well each fills the chip's workgroup slots: 256 CUs hold
// 2 workgroups of the 128 x 128 kernel or 3 of the 64 x 64 one.  Per CU the
// two run at about the same rate with full rounds, and the small tile is
// weighted 0.9 for its extra operand traffic (measured on 512..8192-sized
// squares and 8192 x 1024).
int f32_tile(int64_t M, int64_t N) {
    const int64_t tl = cdiv(M, kF32TileM[0]) * cdiv(N, kF32TileN[0]);
    const int64_t ts = cdiv(M, kF32TileM[1]) * cdiv(N, kF32TileN[1]);
    const double fill_l = (double)tl / (double)(cdiv(tl, 512) * 512);
    const double fill_s = 0.9 * (double)ts / (double)(cdiv(ts, 768) * 768);
    return fill_l >= fill_s ? 0 : 1;
}

// fp32 GEMM (the fp32 matrix cores): row-major operands on the fp32 kernel,
// which needs K in whole 16-element slices, N % 4 == 0 and 16-byte rows.
mg_status gemm_f32(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N, int64_t K,
                   int64_t sam, int64_t sak, int64_t sbk, int64_t sbn, int64_t scm, int64_t scn, mg_dtype in_dtype,
                   mg_dtype out_dtype, bool epi, hipStream_t stream, bool dry = false) {
    if (in_dtype != MG_F32 || out_dtype != MG_F32) return MG_ERR_UNSUPPORTED_DTYPE;
    if (!(sak == 1 || K <= 1) || !(sbn == 1 || N <= 1)) return MG_ERR_UNSUPPORTED_LAYOUT;
    MG_TRY(check_matrix(A, M, K, sam, sak, 4));
    MG_TRY(check_matrix(B, K, N, sbk, sbn, 4));
    MG_TRY(check_matrix(C, M, N, scm, scn, 4));
    if (epi && N > 0 && M > 0 && bias == nullptr) return MG_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return MG_OK;
    if (K % kF32SliceK != 0 || N % 4 != 0) return MG_ERR_UNSUPPORTED_LAYOUT;
    const int tile = f32_tile(M, N);
    const int64_t lim = (int64_t)1 << 31;
    if ((int64_t)kF32TileM[tile] * sam * 4 >= lim || ((int64_t)kF32SliceK * sbk + kF32TileN[tile]) * 4 >= lim)
        return MG_ERR_UNSUPPORTED_LAYOUT;
    KArgs a{};
    a.A = (const uint16_t*)A;  // the fp32 kernel reinterprets the pointers
    a.B = (const uint16_t*)B;
    a.C = (uint16_t*)C;
    a.bias = (const uint16_t*)bias;
    a.M = M; a.N = N; a.K = K;
    a.lda = sam; a.ldb = sbk; a.ldc = scm;
    const int64_t tm = cdiv(M, kF32TileM[tile]), tn = cdiv(N, kF32TileN[tile]);
    if (tm > 0x7fffffff || tn > 0x7fffffff || tm * tn > 0x7fffffff) return MG_ERR_INVALID_ARG;
    const int64_t grid = tm * tn;
    a.tiles_m = (int32_t)tm;
    a.tiles_n = (int32_t)tn;
    a.grid = (int32_t)grid;
    a.group_m = kGroupM;
    a.xcd_remap = 1;
    a.batch = 1;
    if (dry) return MG_OK;
    return launch_f32(tile, epi, a, grid, stream);
}

mg_status gemm_common(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N, int64_t K,
                      int64_t sam, int64_t sak, int64_t sbk, int64_t sbn, int64_t scm, int64_t scn,
                      mg_dtype in_dtype, mg_dtype out_dtype, bool epi, hipStream_t stream, int64_t batch = 1,
                      int64_t sab = 0, int64_t sbb = 0, int64_t scb = 0, bool dry = false) {
    if (M < 0 || N < 0 || K < 0 || batch < 0) return MG_ERR_INVALID_ARG;
    if (in_dtype == MG_F32 || out_dtype == MG_F32) {
        if (batch != 1) return MG_ERR_UNSUPPORTED_DTYPE;
        return gemm_f32(A, B, bias, C, M, N, K, sam, sak, sbk, sbn, scm, scn, in_dtype, out_dtype, epi, stream, dry);
    }
    if (batch == 0) return check_dtype(in_dtype, out_dtype);  // no entries: pointers never used
    if (batch > 1) {
        // entries of A and B may repeat (stride 0); entries of C may not overlap
        if (sab < 0 || sbb < 0 || scb < 0) return MG_ERR_INVALID_ARG;
        if (M > 0 && N > 0 && scb < M * scm) return MG_ERR_UNSUPPORTED_LAYOUT;
        if (sab % 8 != 0 || sbb % 8 != 0 || scb % 8 != 0) return MG_ERR_MISALIGNED;
    }
    MG_TRY(check_dtype(in_dtype, out_dtype));
    // A is row-major (unit stride along K) or given transposed (unit stride
    // along M, i.e. stored [K,M]); likewise B row-major (unit stride along N)
    // or transposed (unit stride along K, stored [N,K]).  The row-major
    // reading wins when both strides are 1 (a single row or column).
    const int ta = (sak == 1 || K <= 1) ? 0 : ((sam == 1 || M <= 1) ? 1 : -1);
    const int tb = (sbn == 1 || N <= 1) ? 0 : ((sbk == 1 || K <= 1) ? 1 : -1);
    if (ta < 0 || tb < 0) return MG_ERR_UNSUPPORTED_LAYOUT;
    MG_TRY(ta ? check_matrix(A, K, M, sak, sam) : check_matrix(A, M, K, sam, sak));
    MG_TRY(tb ? check_matrix(B, N, K, sbn, sbk) : check_matrix(B, K, N, sbk, sbn));
    MG_TRY(check_matrix(C, M, N, scm, scn));
    if (epi && N > 0 && M > 0 && bias == nullptr) return MG_ERR_INVALID_ARG;
    if (M == 0 || N == 0 || batch == 0) return MG_OK;
    const int cfg = select_config(M, N, K, 0, batch);
    if (cfg < 0 || cfg >= kNumConfigs) return MG_ERR_BAD_CONFIG;
    KArgs a{};
    a.A = (const uint16_t*)A;
    a.B = (const uint16_t*)B;
    a.C = (uint16_t*)C;
    a.bias = (const uint16_t*)bias;
    a.M = M; a.N = N; a.K = K;
    a.lda = ta ? sak : sam;  // stride between the stored rows
    a.ldb = tb ? sbn : sbk;
    a.ldc = scm;
    a.batch = (int32_t)(batch > 1 ? batch : 1);
    if (batch > 0x7fffffff) return MG_ERR_INVALID_ARG;
    a.sab = sab; a.sbb = sbb; a.scb = scb;
    a.dry = dry ? 1 : 0;
    return launch(cfg, (int)in_dtype, epi, MODE_DENSE, a, stream, ta, tb);
}

// ---- convolution geometry and im2col -----------------------------------------
struct ConvGeom {
    int64_t OH, OW, M, K, taps;
};

int elem_bytes(mg_dtype dt) { return dt == MG_F16 || dt == MG_BF16 ? 2 : (dt == MG_F32 ? 4 : 0); }

// Checks the shape and derives the output size; the limits keep every index
// of the im2col kernels (32-bit row and column decodes) in range.
mg_status conv_geom(const mg_conv2d_shape* s, ConvGeom& g) {
    if (s == nullptr) return MG_ERR_INVALID_ARG;
    if (s->batch < 0 || s->height < 0 || s->width < 0 || s->in_channels < 0 || s->out_channels < 0)
        return MG_ERR_INVALID_ARG;
    if (s->kernel_h < 1 || s->kernel_w < 1 || s->stride_h < 1 || s->stride_w < 1 || s->dilation_h < 1 ||
        s->dilation_w < 1 || s->pad_h < 0 || s->pad_w < 0)
        return MG_ERR_INVALID_ARG;
    const int64_t lim30 = (int64_t)1 << 30;
    if (s->height >= lim30 || s->width >= lim30 || s->pad_h >= lim30 || s->pad_w >= lim30 ||
        s->kernel_h >= lim30 || s->kernel_w >= lim30 || s->dilation_h >= lim30 || s->dilation_w >= lim30 ||
        s->stride_h >= lim30 || s->stride_w >= lim30 || s->height + 2 * s->pad_h >= lim30 ||
        s->width + 2 * s->pad_w >= lim30)
        return MG_ERR_UNSUPPORTED_LAYOUT;
    const int64_t eh = s->height + 2 * s->pad_h - s->dilation_h * (s->kernel_h - 1) - 1;
    const int64_t ew = s->width + 2 * s->pad_w - s->dilation_w * (s->kernel_w - 1) - 1;
    if (eh < 0 || ew < 0) return MG_ERR_INVALID_ARG;  // the kernel does not fit: empty output
    g.OH = eh / s->stride_h + 1;
    g.OW = ew / s->stride_w + 1;
    const int64_t lim31 = ((int64_t)1 << 31) - 1;
    const int64_t ohw = g.OH * g.OW;  // both < 2^30
    if (ohw > lim31 || (s->batch > 0 && ohw > lim31 / s->batch)) return MG_ERR_UNSUPPORTED_LAYOUT;
    g.M = s->batch * ohw;
    if (s->kernel_h * s->kernel_w > 65535) return MG_ERR_UNSUPPORTED_LAYOUT;
    g.taps = s->kernel_h * s->kernel_w;
    if (s->in_channels >= ((int64_t)1 << 27) / g.taps) return MG_ERR_UNSUPPORTED_LAYOUT;
    g.K = g.taps * s->in_channels;
    return MG_OK;
}

int64_t im2col_ld(int64_t K, int es) {
    const int64_t v = 16 / es;
    return (K + v - 1) / v * v;
}

// The input itself is the GEMM's A for a 1x1 kernel with unit stride and no
// padding, when its channel rows span whole 16-byte chunks.
bool conv_zero_copy(const mg_conv2d_shape* s, int es) {
    return s->kernel_h == 1 && s->kernel_w == 1 && s->stride_h == 1 && s->stride_w == 1 && s->pad_h == 0 &&
           s->pad_w == 0 && (s->in_channels * es) % 16 == 0;
}

// The GEMM gathers its A operand from the image itself (MODE_CONV): 16-bit
// types, an image batch below 2^31 bytes (32-bit load offsets), and a table
// row (the selected or the forced one) with a direct-to-LDS kernel whose K
// slice divides the channel count, so that a slice lies within one tap.
bool conv_implicit(const mg_conv2d_shape* s, const ConvGeom& g, int es) {
    if (es != 2 || s->in_channels <= 0 || s->out_channels <= 0 || g.M <= 0) return false;
    const int64_t lim = ((int64_t)1 << 31) / (2 * s->in_channels);  // pixels that fit
    const int64_t px = s->height * s->width;                           // both < 2^30, batch > 0 here
    if (px > lim || s->batch > lim / px) return false;
    const int cfg = select_config(g.M, s->out_channels, g.K, 0);
    if (cfg < 0 || cfg >= kNumConfigs) return false;
    const mg_config_desc& d = kTable[cfg];
    return d.direct_lds == 1 && d.direct_ksplit == 1 && s->in_channels % d.direct_bk == 0;
}

// Implicit-GEMM convolution: one launch of the selected row's gathering kernel.
mg_status conv_implicit_launch(const mg_conv2d_shape* s, const ConvGeom& g, const void* x, const void* w,
                               int64_t swk, int64_t swn, const void* bias, void* y, mg_dtype dtype,
                               hipStream_t stream) {
    const int64_t N = s->out_channels, K = g.K;
    const int tb = (swn == 1 || N <= 1) ? 0 : ((swk == 1 || K <= 1) ? 1 : -1);
    if (tb < 0) return MG_ERR_UNSUPPORTED_LAYOUT;
    MG_TRY(tb ? check_matrix(w, N, K, swn, swk) : check_matrix(w, K, N, swk, swn));
    MG_TRY(check_matrix(y, g.M, N, N, 1));
    const int cfg = select_config(g.M, N, K, 0);
    if (cfg < 0 || cfg >= kNumConfigs) return MG_ERR_BAD_CONFIG;
    KArgs a{};
    a.A = (const uint16_t*)x;
    a.B = (const uint16_t*)w;
    a.C = (uint16_t*)y;
    a.bias = (const uint16_t*)bias;
    a.M = g.M; a.N = N; a.K = K;
    a.lda = 0;  // unused: rows are gathered
    a.ldb = tb ? swn : swk;
    a.ldc = N;
    a.batch = 1;
    a.conv = ConvArgs{(int32_t)s->height, (int32_t)s->width, (int32_t)s->in_channels, (int32_t)s->kernel_w,
                      (int32_t)s->stride_h, (int32_t)s->stride_w, (int32_t)s->pad_h, (int32_t)s->pad_w,
                      (int32_t)s->dilation_h, (int32_t)s->dilation_w, (int32_t)g.OH, (int32_t)g.OW};
    return launch(cfg, (int)dtype, bias != nullptr, MODE_CONV, a, stream, 0, tb);
}

// Validated arguments; enqueues the im2col kernel.
mg_status launch_im2col(const mg_conv2d_shape* s, const ConvGeom& g, const void* x, void* cols, int64_t ld, int es,
                        hipStream_t stream) {
    if (g.M == 0 || ld == 0) return MG_OK;
    Im2colArgs a{};
    a.x = (const char*)x;
    a.cols = (char*)cols;
    a.H = s->height; a.W = s->width; a.C = s->in_channels;
    a.M = g.M; a.K = g.K; a.ld = ld;
    a.KH = (int32_t)s->kernel_h; a.KW = (int32_t)s->kernel_w;
    a.sh = (int32_t)s->stride_h; a.sw = (int32_t)s->stride_w;
    a.ph = (int32_t)s->pad_h; a.pw = (int32_t)s->pad_w;
    a.dh = (int32_t)s->dilation_h; a.dw = (int32_t)s->dilation_w;
    a.OH = (int32_t)g.OH; a.OW = (int32_t)g.OW;
    const int64_t v = 16 / es;
    const bool tap = g.K > 0 && ld == g.K && s->in_channels % v == 0;
    const int64_t per_row = tap ? s->in_channels / v : ld / v;  // 16-byte chunks per row of one launch
    int64_t rows = 2048 / per_row;
    rows = rows < 1 ? 1 : (rows > kIm2colMaxRows ? kIm2colMaxRows : rows);
    a.rows_per_block = (int32_t)rows;
    // one grid dimension holds at most 2^32 - 1 work-items (reached only by
    // column buffers of several hundred GiB)
    if (cdiv(g.M, rows) * kIm2colThreads > 0xffffffffLL) return MG_ERR_INVALID_ARG;
    const dim3 grid((unsigned)cdiv(g.M, rows), tap ? (unsigned)g.taps : 1u);
    (void)hipGetLastError();
    if (tap) {
        if (es == 2) hipLaunchKernelGGL(im2col_tap_kernel<2>, grid, dim3(kIm2colThreads), 0, stream, a);
        else hipLaunchKernelGGL(im2col_tap_kernel<4>, grid, dim3(kIm2colThreads), 0, stream, a);
    } else {
        if (es == 2) hipLaunchKernelGGL(im2col_elem_kernel<2>, grid, dim3(kIm2colThreads), 0, stream, a);
        else hipLaunchKernelGGL(im2col_elem_kernel<4>, grid, dim3(kIm2colThreads), 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? MG_OK : MG_ERR_HIP;
}

mg_status check_image(const mg_conv2d_shape* s, const void* x) {
    if (s->batch * s->height * s->width * s->in_channels == 0) return MG_OK;  // no extent
    if (x == nullptr) return MG_ERR_INVALID_ARG;
    return aligned16(x) ? MG_OK : MG_ERR_MISALIGNED;
}

}  // namespace

namespace mg {
void note_kernel(int family) { g_last_kernel.store(family); }
}  // namespace mg

extern "C" {

const char* mg_status_string(mg_status status) {
    switch (status) {
        case MG_OK: return "MG_OK";
        case MG_ERR_INVALID_ARG: return "MG_ERR_INVALID_ARG: null pointer with a nonzero extent, or a negative size";
        case MG_ERR_UNSUPPORTED_DTYPE: return "MG_ERR_UNSUPPORTED_DTYPE: types must be fp16 or bf16, in == out";
        case MG_ERR_UNSUPPORTED_LAYOUT: return "MG_ERR_UNSUPPORTED_LAYOUT: inner stride must be 1 and rows must not overlap";
        case MG_ERR_MISALIGNED: return "MG_ERR_MISALIGNED: base pointers must be 16-byte aligned, leading strides multiples of 8";
        case MG_ERR_HIP: return "MG_ERR_HIP: the HIP runtime reported an error at launch";
        case MG_ERR_BAD_CONFIG: return "MG_ERR_BAD_CONFIG: unknown configuration or K step";
    }
    return "unknown mg_status";
}

mg_status mg_gemm(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int64_t stride_am,
                  int64_t stride_ak, int64_t stride_bk, int64_t stride_bn, int64_t stride_cm, int64_t stride_cn,
                  mg_dtype in_dtype, mg_dtype out_dtype, hipStream_t stream) {
    return gemm_common(A, B, nullptr, C, M, N, K, stride_am, stride_ak, stride_bk, stride_bn, stride_cm, stride_cn,
                       in_dtype, out_dtype, false, stream);
}

mg_status mg_gemm_bias_relu(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N, int64_t K,
                            int64_t stride_am, int64_t stride_ak, int64_t stride_bk, int64_t stride_bn,
                            int64_t stride_cm, int64_t stride_cn, mg_dtype in_dtype, mg_dtype out_dtype,
                            hipStream_t stream) {
    return gemm_common(A, B, bias, C, M, N, K, stride_am, stride_ak, stride_bk, stride_bn, stride_cm, stride_cn,
                       in_dtype, out_dtype, true, stream);
}

mg_status mg_gemm_batched(const void* A, const void* B, void* C, int64_t batch, int64_t M, int64_t N, int64_t K,
                          int64_t stride_am, int64_t stride_ak, int64_t stride_bk, int64_t stride_bn,
                          int64_t stride_cm, int64_t stride_cn, int64_t batch_stride_a, int64_t batch_stride_b,
                          int64_t batch_stride_c, mg_dtype in_dtype, mg_dtype out_dtype, hipStream_t stream) {
    return gemm_common(A, B, nullptr, C, M, N, K, stride_am, stride_ak, stride_bk, stride_bn, stride_cm, stride_cn,
                       in_dtype, out_dtype, false, stream, batch, batch_stride_a, batch_stride_b, batch_stride_c);
}

int64_t mg_splitk_choose(int64_t M, int64_t N, int64_t K) {
    // a shape the sweep timed split takes its measured best count; others
    // the count of least modelled time (mg_rates.h: the rows' fitted tile
    // times and the measured rate of writing and reading the fp32
    // partials); a split must win by 5 %, and runs keep at least 256 of K
    if (M <= 0 || N <= 0 || K <= 0) return 1;
    for (const rates::SweptSplit& sw : rates::kSweptSplit)
        if (sw.M == M && sw.N == N && sw.K == K) return sw.splits;
    int64_t best_s = 1;
    double best_t = 0.0;
    for (int64_t s = 1; s <= 64; s *= 2) {
        if (s > 1 && K / s < 256) break;
        const double t = splitk_seconds(M, N, K, s, nullptr);
        if (best_t == 0.0 || t < best_t * 0.95) {
            best_t = t;
            best_s = s;
        }
    }
    return best_s;
}

int64_t mg_prepack_uses_to_pay(int64_t M, int64_t N, int64_t K, mg_dtype dtype) {
    // The layout planner's cost/benefit test ("Using Triton to optimise GEMM
    // across chips", section 3.2: re-lay A out only when the gain exceeds the
    // copy): the gain per call is the modelled time of the chosen row times
    // (1 - packed/plain time ratio measured by the sweep), the cost is the
    // blocking copy (read A, write the blocked copy) at the copy rate the
    // sweep measured.  Returns the number of GEMMs sharing one blocked A
    // after which the copy has paid for itself, or -1 when the blocked
    // layout is not faster on this row.
    (void)dtype;
    if (M <= 0 || N <= 0 || K <= 0) return -1;
    const int cfg = select_config(M, N, K, 0);
    if (cfg < 0 || cfg >= kNumConfigs || cfg >= (int)(sizeof(rates::kPackedRatio) / sizeof(double))) return -1;
    const double ratio = rates::kPackedRatio[cfg];
    if (ratio <= 0.0 || ratio >= 1.0) return -1;
    double t_plain = -1.0;
    for (const rates::RowRate& r : rates::kRows)
        if (r.id == cfg) t_plain = model_seconds(r, tiles_of(r, M, N, 0, 1), K);
    if (t_plain <= 0.0) return -1;
    const int64_t bk = kTable[cfg].bk;
    const double copy = (2.0 * (double)M * (double)K + 2.0 * (double)cdiv(K, bk) * (double)M * (double)bk) /
                        rates::kCopyBytesPerSec;
    const double gain = t_plain * (1.0 - ratio);
    return (int64_t)std::ceil(copy / gain);
}

size_t mg_splitk_workspace_bytes(int64_t M, int64_t N, int64_t splits) {
    if (M <= 0 || N <= 0 || splits <= 0) return 0;
    return (size_t)(splits * M * N) * sizeof(float);
}

}  // extern "C"

namespace {

// Split-K, validation of everything but the workspace (no HIP call).
mg_status splitk_check(const void* A, const void* B, void* C, int64_t splits, int64_t M, int64_t N, int64_t K,
                       int64_t stride_am, int64_t stride_ak, int64_t stride_bk, int64_t stride_bn, int64_t stride_cm,
                       int64_t stride_cn, mg_dtype in_dtype, mg_dtype out_dtype, int& ta, int& tb) {
    if (M < 0 || N < 0 || K < 0 || splits < 1 || splits > 4096) return MG_ERR_INVALID_ARG;
    MG_TRY(check_dtype(in_dtype, out_dtype));
    ta = (stride_ak == 1 || K <= 1) ? 0 : ((stride_am == 1 || M <= 1) ? 1 : -1);
    tb = (stride_bn == 1 || N <= 1) ? 0 : ((stride_bk == 1 || K <= 1) ? 1 : -1);
    if (ta < 0 || tb < 0) return MG_ERR_UNSUPPORTED_LAYOUT;
    MG_TRY(ta ? check_matrix(A, K, M, stride_ak, stride_am) : check_matrix(A, M, K, stride_am, stride_ak));
    MG_TRY(tb ? check_matrix(B, N, K, stride_bn, stride_bk) : check_matrix(B, K, N, stride_bk, stride_bn));
    return check_matrix(C, M, N, stride_cm, stride_cn);
}

// Split-K launch on a validated problem with a workspace of at least
// splits * M * N floats.
mg_status splitk_launch(const void* A, const void* B, void* C, void* workspace, int64_t splits, int64_t M, int64_t N,
                        int64_t K, int64_t stride_am, int64_t stride_ak, int64_t stride_bk, int64_t stride_bn,
                        int64_t stride_cm, mg_dtype in_dtype, int ta, int tb, hipStream_t stream,
                        bool dry = false) {
    const int cfg = select_config_splitk(M, N, K, splits);
    if (cfg < 0 || cfg >= kNumConfigs) return MG_ERR_BAD_CONFIG;
    KArgs a{};
    a.A = (const uint16_t*)A;
    a.B = (const uint16_t*)B;
    a.C = (uint16_t*)C;
    a.M = M; a.N = N; a.K = K;
    a.lda = ta ? stride_ak : stride_am;
    a.ldb = tb ? stride_bn : stride_bk;
    a.ldc = stride_cm;
    a.ws = (float*)workspace;
    a.splits = (int32_t)splits;
    a.dry = dry ? 1 : 0;
    return launch(cfg, (int)in_dtype, false, MODE_SPLITK, a, stream, ta, tb);
}

// ---- split-K without allocation ------------------------------------------------
// The fp32 partials of mg_gemm_splitk_noalloc live in this array: one copy
// per GPU, created when the library's code object is loaded on that GPU and
// held until the process ends.  Host code never uses the name itself (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (nullptr on error).
void* scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

mg_status mg_gemm_splitk(const void* A, const void* B, void* C, void* workspace, size_t workspace_bytes,
                         int64_t splits, int64_t M, int64_t N, int64_t K, int64_t stride_am, int64_t stride_ak,
                         int64_t stride_bk, int64_t stride_bn, int64_t stride_cm, int64_t stride_cn,
                         mg_dtype in_dtype, mg_dtype out_dtype, hipStream_t stream) {
    int ta = 0, tb = 0;
    MG_TRY(splitk_check(A, B, C, splits, M, N, K, stride_am, stride_ak, stride_bk, stride_bn, stride_cm, stride_cn,
                        in_dtype, out_dtype, ta, tb));
    if (M == 0 || N == 0) return MG_OK;
    if (workspace == nullptr || workspace_bytes < mg_splitk_workspace_bytes(M, N, splits))
        return MG_ERR_INVALID_ARG;
    if (!aligned16(workspace)) return MG_ERR_MISALIGNED;
    return splitk_launch(A, B, C, workspace, splits, M, N, K, stride_am, stride_ak, stride_bk, stride_bn, stride_cm,
                         in_dtype, ta, tb, stream);
}

size_t mg_splitk_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

mg_status mg_gemm_splitk_noalloc(const void* A, const void* B, void* C, int64_t splits, int64_t M, int64_t N,
                                 int64_t K, int64_t stride_am, int64_t stride_ak, int64_t stride_bk,
                                 int64_t stride_bn, int64_t stride_cm, int64_t stride_cn, mg_dtype in_dtype,
                                 mg_dtype out_dtype, hipStream_t stream) {
    int ta = 0, tb = 0;
    MG_TRY(splitk_check(A, B, C, splits, M, N, K, stride_am, stride_ak, stride_bk, stride_bn, stride_cm, stride_cn,
                        in_dtype, out_dtype, ta, tb));
    if (M == 0 || N == 0) return MG_OK;
    if (mg_splitk_workspace_bytes(M, N, splits) > kNoAllocScratchBytes) return MG_ERR_INVALID_ARG;
    // the shape checks of the launch itself, still without a HIP call
    MG_TRY(splitk_launch(A, B, C, nullptr, splits, M, N, K, stride_am, stride_ak, stride_bk, stride_bn, stride_cm,
                         in_dtype, ta, tb, stream, /*dry=*/true));
    void* ws = scratch_address();
    if (ws == nullptr) return MG_ERR_HIP;
    return splitk_launch(A, B, C, ws, splits, M, N, K, stride_am, stride_ak, stride_bk, stride_bn, stride_cm,
                         in_dtype, ta, tb, stream);
}

mg_status mg_grouped_gemm(const void* X, const void* W, void* Y, const int32_t* expert_offsets, int64_t E, int64_t T,
                          int64_t N, int64_t K, int64_t stride_xm, int64_t stride_we, int64_t stride_wk,
                          int64_t stride_ym, mg_dtype dtype, hipStream_t stream) {
    if (E < 0 || T < 0 || N < 0 || K < 0 || E > 0x7fffffff || T > 0x7fffffff) return MG_ERR_INVALID_ARG;
    MG_TRY(check_dtype(dtype, dtype));
    if (E == 0 && T > 0) return MG_ERR_INVALID_ARG;
    MG_TRY(check_matrix(X, T, K, stride_xm, 1));
    MG_TRY(check_matrix(Y, T, N, stride_ym, 1));
    if (E > 0 && K > 0 && N > 0) {
        MG_TRY(check_matrix(W, K, N, stride_wk, 1));
        if (E > 1 && stride_we < (K - 1) * stride_wk + N) return MG_ERR_UNSUPPORTED_LAYOUT;
        if (stride_we % 8 != 0) return MG_ERR_MISALIGNED;
    }
    if (T == 0 || N == 0) return MG_OK;
    if (expert_offsets == nullptr) return MG_ERR_INVALID_ARG;
    const int cfg = select_config(T, N, K, E > 0 ? E : 1);
    if (cfg < 0 || cfg >= kNumConfigs) return MG_ERR_BAD_CONFIG;
    KArgs a{};
    a.A = (const uint16_t*)X;
    a.B = (const uint16_t*)W;
    a.C = (uint16_t*)Y;
    a.offsets = expert_offsets;
    a.M = T; a.N = N; a.K = K;
    a.lda = stride_xm; a.ldb = stride_wk; a.ldc = stride_ym;
    a.stride_we = stride_we;
    a.E = (int32_t)E;
    return launch(cfg, (int)dtype, false, MODE_GROUPED, a, stream);
}

size_t mg_prepacked_bytes(int64_t M, int64_t K, int64_t BK, mg_dtype dtype) {
    (void)dtype;
    if (M <= 0 || K <= 0 || BK <= 0) return 0;
    return (size_t)(cdiv(K, BK) * M * BK * 2);
}

int64_t mg_config_bk(int64_t M, int64_t N, int64_t K, mg_dtype dtype) {
    (void)dtype;
    const int cfg = select_config(M, N, K, 0);
    if (cfg < 0 || cfg >= kNumConfigs) return -1;
    return kTable[cfg].bk;
}

mg_status mg_prepack_a(const void* A, void* Ap, int64_t M, int64_t K, int64_t stride_am, int64_t BK, mg_dtype dtype,
                       hipStream_t stream) {
    if (M < 0 || K < 0) return MG_ERR_INVALID_ARG;
    MG_TRY(check_dtype(dtype, dtype));
    if (BK != 32 && BK != 64) return MG_ERR_BAD_CONFIG;
    MG_TRY(check_matrix(A, M, K, stride_am, 1));
    if (M == 0 || K == 0) return MG_OK;
    if (Ap == nullptr) return MG_ERR_INVALID_ARG;
    if (!aligned16(Ap)) return MG_ERR_MISALIGNED;
    const int64_t chunks = cdiv(K, BK) * M * (BK / 8);
    int64_t grid = cdiv(chunks, 256);
    if (grid > 65536) grid = 65536;
    (void)hipGetLastError();
    if (BK == 64)
        hipLaunchKernelGGL((prepack_a_kernel<64>), dim3((unsigned)grid), dim3(256), 0, stream, (const uint16_t*)A,
                           (uint16_t*)Ap, M, K, stride_am);
    else
        hipLaunchKernelGGL((prepack_a_kernel<32>), dim3((unsigned)grid), dim3(256), 0, stream, (const uint16_t*)A,
                           (uint16_t*)Ap, M, K, stride_am);
    return hipGetLastError() == hipSuccess ? MG_OK : MG_ERR_HIP;
}

mg_status mg_gemm_prepacked(const void* Ap, int64_t BK, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                            int64_t stride_bk, int64_t stride_bn, int64_t stride_cm, int64_t stride_cn,
                            mg_dtype dtype, hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0) return MG_ERR_INVALID_ARG;
    MG_TRY(check_dtype(dtype, dtype));
    MG_TRY(check_matrix(B, K, N, stride_bk, stride_bn));
    MG_TRY(check_matrix(C, M, N, stride_cm, stride_cn));
    if (M > 0 && K > 0) {
        if (Ap == nullptr) return MG_ERR_INVALID_ARG;
        if (!aligned16(Ap)) return MG_ERR_MISALIGNED;
    }
    if (M == 0 || N == 0) return MG_OK;
    const int cfg = select_config(M, N, K, 0);
    if (cfg < 0 || cfg >= kNumConfigs) return MG_ERR_BAD_CONFIG;
    if (kTable[cfg].bk != BK) return MG_ERR_BAD_CONFIG;
    KArgs a{};
    a.A = (const uint16_t*)Ap;
    a.B = (const uint16_t*)B;
    a.C = (uint16_t*)C;
    a.M = M; a.N = N; a.K = K;
    a.lda = BK; a.ldb = stride_bk; a.ldc = stride_cm;
    return launch(cfg, (int)dtype, false, MODE_PACKED_A, a, stream);
}

int mg_num_configs(void) { return kNumConfigs; }

mg_status mg_config_info(int id, mg_config_desc* out) {
    if (id < 0 || id >= kNumConfigs) return MG_ERR_BAD_CONFIG;
    if (out == nullptr) return MG_ERR_INVALID_ARG;
    *out = kTable[id];
    return MG_OK;
}

mg_status mg_set_config(int id) {
    if (id < -1 || id >= kNumConfigs) return MG_ERR_BAD_CONFIG;
    g_forced.store(id);
    return MG_OK;
}

int mg_last_config(void) { return g_last.load(); }

mg_status mg_set_raster(int group_m, int xcd_remap) {
    if (group_m == 0 || group_m < -1 || group_m > 256 || xcd_remap < -1 || xcd_remap > 1) return MG_ERR_INVALID_ARG;
    g_group_m.store(group_m);
    g_xcd.store(xcd_remap);
    return MG_OK;
}

int mg_last_kernel(void) { return g_last_kernel.load(); }

int mg_select_config(int64_t M, int64_t N, int64_t K, mg_dtype dtype, int grouped, int64_t batch) {
    (void)dtype;
    return select_config(M, N, K, grouped > 0 ? grouped : 0, grouped > 0 ? 1 : batch);
}

mg_status mg_conv2d_output_hw(const mg_conv2d_shape* shape, int64_t* out_h, int64_t* out_w) {
    ConvGeom g{};
    MG_TRY(conv_geom(shape, g));
    if (out_h) *out_h = g.OH;
    if (out_w) *out_w = g.OW;
    return MG_OK;
}

mg_status mg_im2col(const mg_conv2d_shape* shape, const void* x, void* cols, int64_t ld_cols, mg_dtype dtype,
                    hipStream_t stream) {
    ConvGeom g{};
    MG_TRY(conv_geom(shape, g));
    const int es = elem_bytes(dtype);
    if (es == 0) return MG_ERR_UNSUPPORTED_DTYPE;
    if (ld_cols < g.K || ld_cols >= ((int64_t)1 << 27)) return MG_ERR_UNSUPPORTED_LAYOUT;
    if ((ld_cols * es) % 16 != 0) return MG_ERR_MISALIGNED;
    MG_TRY(check_image(shape, x));
    if (g.M == 0 || ld_cols == 0) return MG_OK;
    if (cols == nullptr) return MG_ERR_INVALID_ARG;
    if (!aligned16(cols)) return MG_ERR_MISALIGNED;
    return launch_im2col(shape, g, x, cols, ld_cols, es, stream);
}

size_t mg_conv2d_workspace_bytes(const mg_conv2d_shape* shape, mg_dtype dtype) {
    ConvGeom g{};
    const int es = elem_bytes(dtype);
    if (es == 0 || conv_geom(shape, g) != MG_OK || conv_zero_copy(shape, es) || conv_implicit(shape, g, es))
        return 0;
    return (size_t)(g.M * im2col_ld(g.K, es) * es);
}

mg_status mg_conv2d(const mg_conv2d_shape* shape, const void* x, const void* w, int64_t stride_wk, int64_t stride_wn,
                    const void* bias, void* y, void* workspace, size_t workspace_bytes, mg_dtype dtype,
                    hipStream_t stream) {
    ConvGeom g{};
    MG_TRY(conv_geom(shape, g));
    const int es = elem_bytes(dtype);
    if (es == 0) return MG_ERR_UNSUPPORTED_DTYPE;
    MG_TRY(check_image(shape, x));
    if (g.M == 0 || shape->out_channels == 0) return MG_OK;
    if (!conv_zero_copy(shape, es) && conv_implicit(shape, g, es))
        return conv_implicit_launch(shape, g, x, w, stride_wk, stride_wn, bias, y, dtype, stream);
    const bool direct = conv_zero_copy(shape, es);
    const int64_t ld = direct ? shape->in_channels : im2col_ld(g.K, es);
    const void* A = direct ? x : workspace;
    if (!direct && g.K > 0) {
        if (workspace == nullptr || workspace_bytes < (size_t)(g.M * ld * es)) return MG_ERR_INVALID_ARG;
        if (!aligned16(workspace)) return MG_ERR_MISALIGNED;
    }
    const int64_t N = shape->out_channels;
    // The GEMM y[M, OC] = cols[M, K] * w[K, OC] (+ bias, ReLU), validated in
    // full before anything is enqueued.
    MG_TRY(gemm_common(A, w, bias, y, g.M, N, g.K, ld, 1, stride_wk, stride_wn, N, 1, dtype, dtype,
                       bias != nullptr, stream, 1, 0, 0, 0, /*dry=*/true));
    if (!direct && g.K > 0) MG_TRY(launch_im2col(shape, g, x, workspace, ld, es, stream));
    return gemm_common(A, w, bias, y, g.M, N, g.K, ld, 1, stride_wk, stride_wn, N, 1, dtype, dtype, bias != nullptr,
                       stream);
}

mg_status mg_attention_scores(const void* Q, const void* K, void* S, int64_t heads, int64_t Lq, int64_t Lk, int64_t d,
                              int64_t stride_qh, int64_t stride_qm, int64_t stride_kh, int64_t stride_kn,
                              int64_t stride_sh, int64_t stride_sm, mg_dtype dtype, hipStream_t stream) {
    if (dtype == MG_F32) return MG_ERR_UNSUPPORTED_DTYPE;
    // S_h[Lq, Lk] = Q_h[Lq, d] * B with B = K_h^T: element (t, j) of B is
    // K_h[j, t], i.e. unit stride along t and stride_kn along j.
    return gemm_common(Q, K, nullptr, S, Lq, Lk, d, stride_qm, 1, 1, stride_kn, stride_sm, 1, dtype, dtype, false,
                       stream, heads, stride_qh, stride_kh, stride_sh);
}

}  // extern "C"
