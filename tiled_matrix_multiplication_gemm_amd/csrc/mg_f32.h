// fp32 GEMM for gfx950: C = A * B with fp32 inputs, the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32) and fp32 output.  The fp32 row of the pages'
// benchmark table (FlagOS cross-chip page, section 3.4, 4096^3 fp32).
//
// Same structure as the 16-bit direct-to-LDS kernel (mg_dlds.h): direct
// 16-byte loads global -> LDS into a ring of K slices with per-slot LDS
// objects, a fence-free barrier per slice, XOR-swizzled chunks.  With 4-byte
// elements the MFMA takes one value of A and of B per lane and k step of 2,
// so the fragment of 8 k values a lane needs for 4 MFMAs is one
// ds_read_b128 of A (4 consecutive k, K-major) and four ds_read_b32 of B
// (one per k-row, N-contiguous): lane l supplies k = 8s + 4 (l / 32) + j to
// MFMA j of step s, in A and B alike.
//
// Preconditions (checked by the host): row-major A and B, K % BK == 0,
// N % 4 == 0, 16-byte aligned rows, and a tile's operand offsets within 31
// bits.  Rows past M and column chunks past N are clamped to the last valid
// ones; what they feed is never stored.
#pragma once

#include "mg_dlds.h"

namespace mg {

template <int BM_, int BN_, int WM_, int WN_, int BK_ = 16, int R_ = 4>
struct F32Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, R = R_;
    static constexpr int NW = WM * WN, NT = NW * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32;
    static constexpr int STEPS = BK / 8;                 // 8 k (4 MFMAs) per step
    static constexpr int ALINE = BK * 4, ACH = BK / 4;   // A: bytes / 16-byte chunks per row
    static constexpr int BLINE = BN * 4, BCH = BN / 4;   // B: bytes / chunks per k-row
    static constexpr int A_BYTES = BM * ALINE, B_BYTES = BK * BLINE, SLOT = A_BYTES + B_BYTES;
    static constexpr int JA = A_BYTES / 1024 / NW, JB = B_BYTES / 1024 / NW;
    static constexpr int LDS_BYTES = R * SLOT;
    static_assert(BK == 16 || BK == 32, "K slice of 16 or 32 fp32");
    static_assert(R >= 3 && R <= 8, "ring of 3..8 slots");
    static_assert(JA * NW * 1024 == A_BYTES && JB * NW * 1024 == B_BYTES, "slice must split evenly over waves");
    static_assert(BCH >= 16, "B k-rows of at least 16 chunks (swizzle spans 8 chunks)");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KB of LDS per CU");
};

// A rows of 64 bytes (BK 16) or 128 bytes (BK 32): the chunk swizzles of the
// 16-bit kernel.  B k-rows: k-rows 4 apart land in the other half of the
// banks, so the two half-waves of a ds_read_b32 (k-rows 4 apart) never meet.
template <int ACH>
__device__ __forceinline__ int swz_a32(int row) { return swz_a<ACH>(row); }
__device__ __forceinline__ int swz_b32(int krow) { return 8 * ((krow >> 2) & 1); }

template <class Cfg, bool EPI>
struct F32Tag {};

template <class Cfg, bool EPI>
__global__ __launch_bounds__(Cfg::NT) void gemm_f32_kernel(const KArgs args) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, FM = Cfg::FM, FN = Cfg::FN;
    constexpr int JA = Cfg::JA, JB = Cfg::JB, STEPS = Cfg::STEPS, R = Cfg::R;
    constexpr int ACH = Cfg::ACH, BCH = Cfg::BCH, ALINE = Cfg::ALINE, BLINE = Cfg::BLINE;
    using Tag = F32Tag<Cfg, EPI>;
    auto slot_ptr = [&](int i) -> char* {  // i is a compile-time constant at every use
        switch (i) {
            case 0: return lds_slot<Cfg::SLOT, 0, Tag>();
            case 1: return lds_slot<Cfg::SLOT, 1, Tag>();
            case 2: return lds_slot<Cfg::SLOT, 2, Tag>();
            case 3: if constexpr (R > 3) return lds_slot<Cfg::SLOT, 3, Tag>(); else return nullptr;
            case 4: if constexpr (R > 4) return lds_slot<Cfg::SLOT, 4, Tag>(); else return nullptr;
            case 5: if constexpr (R > 5) return lds_slot<Cfg::SLOT, 5, Tag>(); else return nullptr;
            case 6: if constexpr (R > 6) return lds_slot<Cfg::SLOT, 6, Tag>(); else return nullptr;
            default: if constexpr (R > 7) return lds_slot<Cfg::SLOT, 7, Tag>(); else return nullptr;
        }
    };
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

    const unsigned wg = tile_block<Cfg::NT>();
    if (wg >= (unsigned)args.grid) return;
    int logical = args.xcd_remap ? xcd_logical((int)wg, args.grid) : (int)wg;
    const float* Ag = (const float*)args.A;
    const float* Bg = (const float*)args.B;
    float* Cg = (float*)args.C;
    int pm, pn;
    grouped_order(logical, args.tiles_m, args.tiles_n, args.group_m, pm, pn);
    const int64_t M = args.M, N = args.N, K = args.K;
    const int64_t m0 = (int64_t)pm * BM, n0 = (int64_t)pn * BN;
    const int nk = (int)(K / BK);

    // ---- direct-load offsets (bytes from the tile's slice base) ---------
    uint32_t offA_g[JA], offB_g[JB];
#pragma unroll
    for (int j = 0; j < JA; ++j) {
        const int q = wave * JA + j;
        const int row = q * (1024 / ALINE) + lane / ACH;
        const int c = (lane % ACH) ^ swz_a32<ACH>(row);
        const int64_t r = (m0 + row < M ? row : M - 1 - m0);
        offA_g[j] = (uint32_t)((r * args.lda + 4 * c) * 4);
    }
#pragma unroll
    for (int j = 0; j < JB; ++j) {
        const int q = wave * JB + j;
        const int krow = q * (1024 / BLINE) + lane / BCH;
        const int c = (lane % BCH) ^ swz_b32(krow);
        const int64_t cn = (n0 + 4 * c <= N - 4) ? 4 * c : N - 4 - n0;
        offB_g[j] = (uint32_t)((krow * args.ldb + cn) * 4);
    }
    const char* baseA = (const char*)(Ag + m0 * args.lda);
    const char* baseB = (const char*)(Bg + n0);
    const int64_t stepA = (int64_t)BK * 4, stepB = (int64_t)BK * args.ldb * 4;
    auto issue = [&](int kt, int slot) {
        const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(baseA + kt * stepA);
        const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(baseB + kt * stepB);
        char* sa = slot_ptr(slot);
        char* sb = sa + Cfg::A_BYTES;
#pragma unroll
        for (int j = 0; j < JA; ++j) direct_load16(ra, offA_g[j], (lds_void_t*)(sa + (wave * JA + j) * 1024));
#pragma unroll
        for (int j = 0; j < JB; ++j) direct_load16(rb, offB_g[j], (lds_void_t*)(sb + (wave * JB + j) * 1024));
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // ---- fragments: A one b128 per row block, B four b32 per column block
    const int h = lane >> 5;
    struct Frags {
        f32x4 a[FM], b[FN];
    };
    auto read_frags = [&](Frags& f, int slot, int s) {
        const char* sa = slot_ptr(slot);
        const char* sb = sa + Cfg::A_BYTES;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * Cfg::WTM + i * 32 + (lane & 31);
            const int c = (2 * s + h) ^ swz_a32<ACH>(row);
            f.a[i] = *(const __attribute__((address_space(3))) f32x4*)(sa + row * ALINE + c * 16);
        }
#pragma unroll
        for (int jb = 0; jb < FN; ++jb) {
            const int col = wn * Cfg::WTN + jb * 32 + (lane & 31);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int krow = 8 * s + 4 * h + j;
                f.b[jb][j] = *(const __attribute__((address_space(3))) float*)(
                    sb + krow * BLINE + (((col >> 2) ^ swz_b32(krow)) * 16) + (col & 3) * 4);
            }
        }
    };
    // B first: the accumulators hold C transposed (as in mg_dlds.h)
    auto mfma_step = [&](const Frags& f) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int jb = 0; jb < FN; ++jb)
                    acc[i][jb] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.b[jb][j], f.a[i][j], acc[i][jb], 0, 0, 0);
    };

    // ---- K loop: ring of R slots, slice t in slot t % R, one barrier per
    // slice; after it, slice t+R-1 refills the slot of slice t-1 (all of
    // whose reads fed MFMAs before the barrier).
    constexpr int L = JA + JB;
    Frags F0, F1;
    auto slice = [&](int t, int u) {
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            Frags& cur = (s & 1) ? F1 : F0;
            Frags& nxt = (s & 1) ? F0 : F1;
            if (s + 1 < STEPS) {
                read_frags(nxt, u, s + 1);
            } else {
                if (t + R - 2 <= nk - 1) wait_vmcnt<L * (R - 3)>();
                else wait_vmcnt<0>();
                ring_barrier();
                if (t + R - 1 < nk) issue(t + R - 1, (u + R - 1) % R);
                if (t + 1 < nk) read_frags(nxt, (u + 1) % R, 0);
            }
            mfma_step(cur);
        }
    };
    if (nk > 0) {
        const int pre = nk < R - 1 ? nk : R - 1;
        for (int t = 0; t < pre; ++t) issue(t, t);
        if (pre == R - 1) wait_vmcnt<L * (R - 2)>();
        else wait_vmcnt<0>();
        ring_barrier();
        read_frags(F0, 0, 0);
        for (int trip = 0; trip < nk; trip += R) {
#pragma unroll
            for (int u = 0; u < R; ++u) {
                if (trip + u >= nk) break;
                slice(trip + u, u);
            }
        }
    }

    // ---- epilogue: 4 adjacent fp32 outputs per lane and register group
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t row = m0 + wm * Cfg::WTM + i * 32 + (lane & 31);
#pragma unroll
        for (int jb = 0; jb < FN; ++jb) {
            const int64_t col0 = n0 + wn * Cfg::WTN + jb * 32 + 4 * h;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t col = col0 + 8 * q;
                f32x4 v = {acc[i][jb][4 * q], acc[i][jb][4 * q + 1], acc[i][jb][4 * q + 2], acc[i][jb][4 * q + 3]};
                if constexpr (EPI) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float bt = (col + t < N) ? ((const float*)args.bias)[col + t] : 0.0f;
                        v[t] = v[t] + bt;
                        v[t] = (v[t] > 0.0f) ? v[t] : 0.0f;
                    }
                }
                if (row < M && col < N) store_out((f32x4*)(Cg + row * args.ldc + col), v);
            }
        }
    }
}

}  // namespace mg
