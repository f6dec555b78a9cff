// Device code of the tiled GEMM: one workgroup computes one BM x BN output
// tile with 32x32x16 MFMA instructions, streaming BK-wide slices of A and B
// through a two-buffer LDS ring.
//
// Method (from the pages): output tiling with a K loop that accumulates in
// fp32 ("Using Triton to optimise GEMM across chips", sections 2.1-2.2),
// multi-buffering so the loads of slice i+1 overlap the math of slice i
// (same page, section 2.2), 128-bit vector loads and XOR-swizzled shared
// memory against bank conflicts (FlagOS cross-chip page, sections 2.3-2.4),
// grouped tile order for L2 reuse (Gluon matmul example; "Triton study
// notes", section 2.3.7), the fused bias + ReLU epilogue (yfxerp page,
// section 3.4) and the blocked A layout (yfxerp page, section 3.2).
//
// gfx950 specifics: 64-lane waves; v_mfma_f32_32x32x16_{f16,bf16}; 160 KB of
// LDS per CU; workgroups dispatched round-robin over 8 XCDs, each with its
// own L2, so consecutive tiles are remapped onto one XCD.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum { DT_F16 = 0, DT_BF16 = 1 };
enum { MODE_DENSE = 0, MODE_PACKED_A = 1, MODE_GROUPED = 2, MODE_SPLITK = 3, MODE_CONV = 4 };

// Implicit-GEMM convolution (MODE_CONV): A is the im2col matrix of an NHWC
// image batch, gathered by the loads themselves.  Output row m = (n OH + oh)
// OW + ow; column k = (kh KW + kw) C + c.
struct ConvArgs {
    int32_t H, W, C, KW;
    int32_t sh, sw, ph, pw, dh, dw;
    int32_t OH, OW;
};

struct KArgs {
    const uint16_t* A;       // dense: A; packed: blocked A; grouped: X
    const uint16_t* B;       // dense: B; grouped: W (expert 0)
    uint16_t* C;             // dense: C; grouped: Y
    const uint16_t* bias;    // fused epilogue only
    const int32_t* offsets;  // grouped only: E+1 row offsets (device)
    int64_t M, N, K;         // grouped: M = T
    int64_t lda, ldb, ldc;   // row strides (elements)
    int64_t stride_we;       // grouped: elements between experts' weights
    int32_t E;
    int32_t tiles_m, tiles_n;
    int32_t batch;           // dense: batch entries (1 for a single GEMM)
    int64_t sab, sbb, scb;   // dense: elements between batch entries of A, B, C
    float* ws;               // split-K: fp32 partial products [splits][M][N]
    int32_t splits;          // split-K: K ranges (contiguous runs of K slices)
    int32_t group_m;
    int32_t xcd_remap;
    int32_t dry;             // host only: 1 = validate the launch, enqueue nothing
    int32_t grid;            // workgroups that hold tiles (grouped: an upper bound)
    ConvArgs conv;           // MODE_CONV only
};

// A dispatch counts at most 2^32 - 1 work-items in each grid dimension, so a
// tile launch of more workgroups than that allows in x is laid out as rows
// of tile_row(NT) workgroups (a multiple of 8, one per XCD) over gridDim.y.
// Workgroup ids are linear, x fastest (the order the dispatcher hands them
// out); the ids past the tile count in the last row return at once.  The
// padded count stays below 2^32 since the host keeps the tile count below
// 2^31.  The row width depends on the workgroup size alone, so the kernels
// take it as a constant instead of reading the grid's shape.
__host__ __device__ constexpr unsigned tile_row(int nt) { return (0xffffffffu / (unsigned)nt) & ~7u; }
inline dim3 tile_grid(int64_t grid, int nt) {
    const int64_t row = tile_row(nt);
    if (grid <= row) return dim3((unsigned)grid);
    return dim3((unsigned)row, (unsigned)((grid + row - 1) / row));
}
template <int NT>
__device__ __forceinline__ unsigned tile_block() { return blockIdx.x + blockIdx.y * tile_row(NT); }

// Grouped GEMM: which tile workgroup `logical` computes.  Tiles run expert by
// expert; within an expert, column slab by column slab, with the expert's row
// tiles of one slab adjacent.  Consecutive workgroups therefore share the
// expert's X rows (which stay in L2 across its column slabs) and the row
// tiles of a slab share its W columns.  Offsets are clamped into [0, T] so
// that malformed offsets cannot send a workgroup outside X or Y.
// grouped_tiles() counts the tiles: the host sizes the grid for the worst
// case (it does not read the device offsets), and the XCD renumbering must
// spread the real tiles, not the grid, over the 8 XCDs.
//
// The offsets as a wave reads them: with fewer than 64 experts one vector
// load puts offsets[e] in lane e and every lookup below is a v_readlane, so
// the walk over the experts waits on memory once instead of once per expert.
struct GroupOffsets {
    int v;          // lane e: offsets[e] (when in_lanes)
    bool in_lanes;  // E < 64
};
__device__ __forceinline__ GroupOffsets load_group_offsets(const KArgs& args) {
    GroupOffsets g;
    g.in_lanes = args.E < 64;
    const int lane = (int)(threadIdx.x & 63);
    g.v = (g.in_lanes && lane <= args.E) ? args.offsets[lane] : 0;
    return g;
}
// The walk over the experts, with `off(e)` giving offsets[e].
template <int BM, class Off>
__device__ __forceinline__ int grouped_tiles_walk(const KArgs& args, Off off) {
    const int T = (int)args.M;
    int total = 0;
    int a = off(0);
    a = a < 0 ? 0 : (a > T ? T : a);
    for (int e = 0; e < args.E; ++e) {
        int b = off(e + 1);
        b = b < a ? a : (b > T ? T : b);
        total += (int)(((unsigned)(b - a) + (BM - 1u)) / BM);  // unsigned: b - a may reach 2^31 - 1
        a = b;
    }
    return total * args.tiles_n;
}
template <int BM, class Off>
__device__ __forceinline__ bool grouped_tile_walk(const KArgs& args, Off off, int logical, int& e, int& r0,
                                                  int& rows, int& pm, int& pn) {
    const int T = (int)args.M;
    int base = 0;
    int a = off(0);
    a = a < 0 ? 0 : (a > T ? T : a);
    for (e = 0; e < args.E; ++e) {
        int b = off(e + 1);
        b = b < a ? a : (b > T ? T : b);
        const int mt = (int)(((unsigned)(b - a) + (BM - 1u)) / BM);
        const int cnt = mt * args.tiles_n;
        if (logical < base + cnt) {
            const int local = logical - base;
            pn = local / mt;
            pm = local % mt;
            r0 = a;
            rows = b - a;
            return true;
        }
        base += cnt;
        a = b;
    }
    return false;
}
// One walk per source of the offsets, chosen outside the loop (a select
// inside it would issue the memory load on every step anyway).
template <int BM>
__device__ __forceinline__ int grouped_tiles(const KArgs& args, const GroupOffsets& go) {
    if (go.in_lanes) return grouped_tiles_walk<BM>(args, [&](int e) { return __builtin_amdgcn_readlane(go.v, e); });
    return grouped_tiles_walk<BM>(args, [&](int e) { return args.offsets[e]; });
}
template <int BM>
__device__ __forceinline__ bool grouped_tile(const KArgs& args, const GroupOffsets& go, int logical, int& e, int& r0,
                                             int& rows, int& pm, int& pn) {
    if (go.in_lanes)
        return grouped_tile_walk<BM>(args, [&](int i) { return __builtin_amdgcn_readlane(go.v, i); }, logical, e, r0,
                                     rows, pm, pn);
    return grouped_tile_walk<BM>(args, [&](int i) { return args.offsets[i]; }, logical, e, r0, rows, pm, pn);
}

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NT = WM * WN * 64;            // threads per workgroup
    static constexpr int KC = BK / 8;                  // 16-byte chunks per tile row
    static constexpr int WTM = BM / WM, WTN = BN / WN; // output of one wave
    static constexpr int FM = WTM / 32, FN = WTN / 32; // MFMA tiles per wave
    static constexpr int A_CHUNKS = BM * KC;           // 16-byte chunks per stage
    static constexpr int B_CHUNKS = BN * KC;
    static constexpr int A_PER_THREAD = (A_CHUNKS + NT - 1) / NT;
    static constexpr int B_BLOCKS = (BK / 8) * (BN / 8); // 8x8 element blocks of B
    static constexpr int B_PER_THREAD = (B_BLOCKS + NT - 1) / NT;
    static constexpr int STAGES = 2;
    static constexpr int LDS_BYTES = STAGES * (A_CHUNKS + B_CHUNKS) * 16;
    static_assert(BK == 32 || BK == 64, "K step must be 32 or 64");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of the 32x32 MFMA tile");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KB of LDS per CU");
};

// XOR swizzle of the 16-byte chunk index within an LDS tile row.  Both
// access patterns of a stage are kept free of bank conflicts: the MFMA
// operand reads (32 consecutive rows, one chunk column) and the transposed
// B writes (rows 8 apart).
template <int KC>
__device__ __forceinline__ int swz(int row) {
    if constexpr (KC == 8) return (row ^ (row >> 3)) & 7;
    else return ((row >> 1) ^ (row >> 3)) & 3;
}

// 16-byte chunk of which only the first `valid` (0..8) elements exist; the
// rest read as +0.0.
__device__ __forceinline__ u32x4 load_partial(const uint16_t* p, int valid) {
    u32x4 v;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t lo = (2 * d < valid) ? (uint32_t)p[2 * d] : 0u;
        uint32_t hi = (2 * d + 1 < valid) ? (uint32_t)p[2 * d + 1] : 0u;
        v[d] = lo | (hi << 16);
    }
    return v;
}

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (DT == DT_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ float to_float(uint16_t bits) {
    if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, bits);
    else return __builtin_bit_cast(float, (uint32_t)bits << 16);
}

// fp32 -> fp16 / bf16, round to nearest even (the hardware conversions).
template <int DT>
__device__ __forceinline__ uint16_t from_float(float v) {
    if constexpr (DT == DT_F16) return __builtin_bit_cast(uint16_t, (_Float16)v);
    else return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Stores of output tiles: written once and not read again by the kernel,
// they go out as nontemporal (streaming) stores, which spares the caches'
// lines for the operands (attention scores, 1 GiB of output: 0.378 ->
// 0.288 ms; 8192^3 0.788 -> 0.780 ms; grouped MoE 0.1075 -> 0.1057 ms, same
// process).
template <class T>
__device__ __forceinline__ void store_out(T* p, const T& v) {
    __builtin_nontemporal_store(v, p);
}

// Workgroups are handed to the 8 XCDs round-robin; renumber them so that
// each XCD receives one contiguous range of logical tile ids.
__device__ __forceinline__ int xcd_logical(int b, int total) {
    const int X = 8;
    int xcd = b % X, local = b / X;
    int q = total / X, r = total % X;
    return (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Dense and batched GEMM: batch entry of workgroup `logical`, whose tile index
// within the entry is returned in `logical`; the operands are advanced to
// the entry.  Entries are contiguous ranges of workgroups, so each XCD works
// on whole tiles of few entries.
__device__ __forceinline__ void batch_entry(const KArgs& args, int& logical, const uint16_t*& A, const uint16_t*& B,
                                            uint16_t*& C) {
    const int per = args.tiles_m * args.tiles_n;
    const int b = logical / per;
    logical -= b * per;
    A += (int64_t)b * args.sab;
    B += (int64_t)b * args.sbb;
    C += (int64_t)b * args.scb;
}

// Grouped tile order: GROUP_M tile rows at a time, column by column within
// the group (the Gluon matmul example's program-id mapping).
// group_m is clamped to tiles_m (one group either way), which keeps
// group_m * tiles_n within the grid's tile count and so within 31 bits.
__device__ __forceinline__ void grouped_order(int pid, int tiles_m, int tiles_n, int group_m, int& pm, int& pn) {
    group_m = min(group_m, tiles_m);
    int per_group = group_m * tiles_n;
    int group = pid / per_group;
    int first = group * group_m;
    int rows = min(tiles_m - first, group_m);
    int local = pid - group * per_group;
    pm = first + local % rows;
    pn = local / rows;
}

template <class Cfg, int DT, bool EPI, int MODE>
__global__ __launch_bounds__(Cfg::NT) void gemm_tile_kernel(const KArgs args) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, KC = Cfg::KC;
    constexpr int NT = Cfg::NT, FM = Cfg::FM, FN = Cfg::FN;
    __shared__ u32x4 smem[Cfg::STAGES * (Cfg::A_CHUNKS + Cfg::B_CHUNKS)];
    u32x4* const sA = smem;                                      // [STAGES][BM][KC]
    u32x4* const sB = smem + Cfg::STAGES * Cfg::A_CHUNKS;        // [STAGES][BN][KC]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

    // ---- which tile -------------------------------------------------------
    const unsigned wg = tile_block<NT>();
    int total = args.grid;
    [[maybe_unused]] GroupOffsets go{0, false};
    if constexpr (MODE == MODE_GROUPED) {
        go = load_group_offsets(args);
        total = grouped_tiles<BM>(args, go);
    }
    if (wg >= (unsigned)total) return;
    int logical = args.xcd_remap ? xcd_logical((int)wg, total) : (int)wg;
    const uint16_t* Ag = args.A;
    const uint16_t* Bg = args.B;
    uint16_t* Cg = args.C;
    int64_t M = args.M;
    int pm, pn;
    if constexpr (MODE == MODE_GROUPED) {
        int e, r0, rows;
        if (!grouped_tile<BM>(args, go, logical, e, r0, rows, pm, pn)) return;
        M = rows;
        Ag += (int64_t)r0 * args.lda;
        Bg += (int64_t)e * args.stride_we;
        Cg += (int64_t)r0 * args.ldc;
    } else {
        if constexpr (MODE == MODE_DENSE) batch_entry(args, logical, Ag, Bg, Cg);
        grouped_order(logical, args.tiles_m, args.tiles_n, args.group_m, pm, pn);
    }
    const int64_t N = args.N, K = args.K;
    const int64_t m0 = (int64_t)pm * BM, n0 = (int64_t)pn * BN;
    const bool interior = (m0 + BM <= M) && (n0 + BN <= N);
    const int nk = (int)((K + BK - 1) / BK);
    const bool k_ragged = (K % BK) != 0;

    // ---- per-thread load slots -------------------------------------------
    u32x4 ra[Cfg::A_PER_THREAD];
    u32x4 rb[Cfg::B_PER_THREAD][8];

    auto load_A = [&](int kt, bool check) {
#pragma unroll
        for (int q = 0; q < Cfg::A_PER_THREAD; ++q) {
            const int c = q * NT + tid;
            if (Cfg::A_CHUNKS % NT != 0 && c >= Cfg::A_CHUNKS) break;
            const int row = c / KC, kc = c % KC;
            int64_t gm = m0 + row;
            if (gm > M - 1) gm = M - 1;   // rows past M only feed rows that are never stored
            const int64_t k = (int64_t)kt * BK + kc * 8;
            if constexpr (MODE == MODE_PACKED_A) {
                // blocked layout: the K tail is already zero-padded
                ra[q] = *(const u32x4*)(Ag + ((int64_t)kt * M + gm) * BK + kc * 8);
            } else {
                const uint16_t* p = Ag + gm * args.lda + k;
                if (!check || k + 8 <= K) ra[q] = *(const u32x4*)p;
                else ra[q] = load_partial(p, (int)(K - k > 0 ? K - k : 0));
            }
        }
    };

    auto load_B = [&](int kt, bool check) {
#pragma unroll
        for (int q = 0; q < Cfg::B_PER_THREAD; ++q) {
            const int b = q * NT + tid;
            if (Cfg::B_BLOCKS % NT != 0 && b >= Cfg::B_BLOCKS) break;
            const int nb = b % (BN / 8), kb = b / (BN / 8);
            const int64_t n = n0 + nb * 8;
            const int64_t kbase = (int64_t)kt * BK + kb * 8;
            const uint16_t* p = Bg + kbase * args.ldb + n;
            if (!check) {
#pragma unroll
                for (int j = 0; j < 8; ++j) rb[q][j] = *(const u32x4*)(p + j * args.ldb);
            } else {
                const int nvalid = (int)(N - n >= 8 ? 8 : (N - n > 0 ? N - n : 0));
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (kbase + j < K && nvalid == 8) rb[q][j] = *(const u32x4*)(p + j * args.ldb);
                    else if (kbase + j < K) rb[q][j] = load_partial(p + j * args.ldb, nvalid);
                    else rb[q][j] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    };

    auto store_stage = [&](int stage) {
        u32x4* a = sA + stage * Cfg::A_CHUNKS;
        u32x4* bs = sB + stage * Cfg::B_CHUNKS;
#pragma unroll
        for (int q = 0; q < Cfg::A_PER_THREAD; ++q) {
            const int c = q * NT + tid;
            if (Cfg::A_CHUNKS % NT != 0 && c >= Cfg::A_CHUNKS) break;
            const int row = c / KC, kc = c % KC;
            a[row * KC + (kc ^ swz<KC>(row))] = ra[q];
        }
#pragma unroll
        for (int q = 0; q < Cfg::B_PER_THREAD; ++q) {
            const int b = q * NT + tid;
            if (Cfg::B_BLOCKS % NT != 0 && b >= Cfg::B_BLOCKS) break;
            const int nb = b % (BN / 8), kb = b / (BN / 8);
            // 8x8 transpose in registers: column i of the block becomes one
            // K-contiguous chunk of row n = 8*nb + i of the LDS B tile.
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                u32x4 t;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t x = rb[q][2 * d][i >> 1], y = rb[q][2 * d + 1][i >> 1];
                    t[d] = (i & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
                }
                const int n = nb * 8 + i;
                bs[n * KC + (kb ^ swz<KC>(n))] = t;
            }
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto compute_stage = [&](int stage) {
        const u32x4* a = sA + stage * Cfg::A_CHUNKS;
        const u32x4* bs = sB + stage * Cfg::B_CHUNKS;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int kc = 2 * s + (lane >> 5);
            u32x4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * Cfg::WTM + i * 32 + (lane & 31);
                fa[i] = a[row * KC + (kc ^ swz<KC>(row))];
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = wn * Cfg::WTN + j * 32 + (lane & 31);
                fb[j] = bs[n * KC + (kc ^ swz<KC>(n))];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<DT>(fa[i], fb[j], acc[i][j]);
        }
    };

    if (nk > 0) {
        const bool check0 = !interior || (nk == 1 && k_ragged);
        load_A(0, check0);
        load_B(0, check0);
        store_stage(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) {
                const bool check = !interior || (kt + 2 == nk && k_ragged);
                load_A(kt + 1, check);
                load_B(kt + 1, check);
            }
            compute_stage(cur);
            if (more) store_stage(cur ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogue: (bias, ReLU), one rounding, masked stores --------------
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t col = n0 + wn * Cfg::WTN + j * 32 + (lane & 31);
        float bj = 0.0f;
        if constexpr (EPI) bj = (col < N) ? to_float<DT>(args.bias[col]) : 0.0f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * Cfg::WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                float v = acc[i][j][r];
                if constexpr (EPI) {
                    v = v + bj;
                    v = (v > 0.0f) ? v : 0.0f;
                }
                if (row < M && col < N) Cg[row * args.ldc + col] = from_float<DT>(v);
            }
        }
    }
}

// Blocked re-layout of A: Ap[kb][m][kk] = A[m][kb*BK + kk] (zero past K).
// One thread per 16-byte chunk of Ap.
template <int BK>
__global__ __launch_bounds__(256) void prepack_a_kernel(const uint16_t* __restrict__ A, uint16_t* __restrict__ Ap,
                                                        int64_t M, int64_t K, int64_t lda) {
    constexpr int KC = BK / 8;
    const int64_t nkb = (K + BK - 1) / BK;
    const int64_t total = nkb * M * KC;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total; c += (int64_t)gridDim.x * 256) {
        const int kc = (int)(c % KC);
        const int64_t m = (c / KC) % M;
        const int64_t kb = c / (KC * M);
        const int64_t k = kb * BK + kc * 8;
        const uint16_t* p = A + m * lda + k;
        u32x4 v;
        if (k + 8 <= K) v = *(const u32x4*)p;
        else v = load_partial(p, (int)(K - k > 0 ? K - k : 0));
        *(u32x4*)(Ap + c * 8) = v;
    }
}

}  // namespace mg
