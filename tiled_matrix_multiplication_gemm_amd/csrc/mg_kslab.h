// Small-tile kernel for gfx950 with the K dimension split across the waves
// of a workgroup.
//
// When the output holds too few large tiles to occupy 256 CUs (a 1024 x 1024
// output is 256 tiles of 64 x 64), each tile is small and its K loop long.
// With one 32 x 32 MFMA tile per wave, a k16 step is a single MFMA, far too
// little work to cover the latency of the LDS reads that feed it, and the
// per-slice workgroup barriers add more.  Here every wave of the workgroup
// owns the whole BM x BN tile but only every NW-th BK slice of K: it loads its
// own slices into a private LDS ring with direct global->LDS loads, waits
// only for its own loads (no barrier anywhere in the K loop), runs FM*FN
// MFMAs per k16 step, and at the end the NW partial sums are added through
// LDS before the epilogue.  The sum over K is thereby split into NW
// interleaved partial sums in fp32 (the pages fix only fp32 accumulation,
// not its order).
//
// Loads, swizzles and fragment reads are those of the direct-to-LDS kernel
// (mg_dlds.h).  Preconditions (checked by the host): K % BK == 0, N % 8 == 0,
// tile offsets fit in 31 bits.
#pragma once

#include "mg_dlds.h"

namespace mg {

template <int BM_, int BN_, int NW_, int BK_, int RW_>
struct SlabCfg {
    static constexpr int BM = BM_, BN = BN_, NW = NW_, BK = BK_, RW = RW_;
    static constexpr int NT = NW * 64;
    static constexpr int FM = BM / 32, FN = BN / 32, Q = FM * FN;  // MFMA tiles of the output tile
    static constexpr int STEPS = BK / 16;
    static constexpr int AROW = BK * 2, ACH = BK / 8;
    static constexpr int A_BYTES = BM * AROW;
    static constexpr int B_BYTES = BK * BN * 2;
    static constexpr int SLOT = A_BYTES + B_BYTES;    // one slice of one wave
    static constexpr int JA = A_BYTES / 1024, JB = B_BYTES / 1024;  // 1 KB loads per slice (one wave)
    static constexpr int OBJ = NW * SLOT;             // one ring slot of every wave
    static constexpr int LDS_BYTES = RW * OBJ;
    static constexpr int BCH = BN / 8;
    static constexpr int WM = 1, WN = 1, STAGES = RW;  // for the configuration table
    static_assert(BK == 32 || BK == 64, "K slice must be 32 or 64");
    static_assert(RW >= 2 && RW <= 8, "ring of 2..8 slots per wave");
    static_assert(JA * 1024 == A_BYTES && JB * 1024 == B_BYTES, "slice must be whole 1 KB loads");
    static_assert((JA + JB) * (RW - 1) < 64, "outstanding loads must fit the 6-bit vmcnt");
    static_assert(Q <= RW && 4096 <= SLOT, "partial sums are staged in the ring slots");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KB of LDS per CU");
};

template <class Cfg, int DT, bool EPI>
struct SlabTag {};

template <class Cfg, int DT, bool EPI>
__global__ __launch_bounds__(Cfg::NT) void gemm_kslab_kernel(const KArgs args) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NW = Cfg::NW, RW = Cfg::RW;
    constexpr int FM = Cfg::FM, FN = Cfg::FN, JA = Cfg::JA, JB = Cfg::JB, BCH = Cfg::BCH;
    constexpr int ACH = Cfg::ACH, AROW = Cfg::AROW, STEPS = Cfg::STEPS;
    using Tag = SlabTag<Cfg, DT, EPI>;
    auto obj = [&](int i) -> char* {  // ring slot objects; i is a compile-time constant at every use
        switch (i) {
            case 0: return lds_slot<Cfg::OBJ, 0, Tag>();
            case 1: return lds_slot<Cfg::OBJ, 1, Tag>();
            case 2: if constexpr (RW > 2) return lds_slot<Cfg::OBJ, 2, Tag>(); else return nullptr;
            case 3: if constexpr (RW > 3) return lds_slot<Cfg::OBJ, 3, Tag>(); else return nullptr;
            case 4: if constexpr (RW > 4) return lds_slot<Cfg::OBJ, 4, Tag>(); else return nullptr;
            case 5: if constexpr (RW > 5) return lds_slot<Cfg::OBJ, 5, Tag>(); else return nullptr;
            case 6: if constexpr (RW > 6) return lds_slot<Cfg::OBJ, 6, Tag>(); else return nullptr;
            default: if constexpr (RW > 7) return lds_slot<Cfg::OBJ, 7, Tag>(); else return nullptr;
        }
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const unsigned wg = tile_block<Cfg::NT>();
    if (wg >= (unsigned)args.grid) return;
    int logical = args.xcd_remap ? xcd_logical((int)wg, args.grid) : (int)wg;
    const uint16_t* Ag = args.A;
    const uint16_t* Bg = args.B;
    uint16_t* Cg = args.C;
    batch_entry(args, logical, Ag, Bg, Cg);
    int pm, pn;
    grouped_order(logical, args.tiles_m, args.tiles_n, args.group_m, pm, pn);
    const int64_t M = args.M, N = args.N, K = args.K;
    const int64_t m0 = (int64_t)pm * BM, n0 = (int64_t)pn * BN;
    const int nk = (int)(K / BK);
    const int mine = nk > wave ? (nk - wave + NW - 1) / NW : 0;  // this wave's slices: wave, wave+NW, ...

    // per-lane source offsets (as in the direct-to-LDS kernel, one wave per slice)
    uint32_t offA_g[JA];
#pragma unroll
    for (int j = 0; j < JA; ++j) {
        const int row = j * (1024 / AROW) + lane / ACH;
        const int c = (lane % ACH) ^ swz_a<ACH>(row);
        const int64_t r = (m0 + row < M ? row : M - 1 - m0);
        offA_g[j] = (uint32_t)((r * args.lda + 8 * c) * 2);
    }
    uint32_t offB_g[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) {
        const int krow = j * (512 / BN) + (8 * lane) / BN;
        const int c = (lane % BCH) ^ swz_b<BCH>(krow);
        const int64_t cn = (n0 + 8 * c <= N - 8) ? 8 * c : N - 8 - n0;
        offB_g[j] = (uint32_t)((krow * args.ldb + cn) * 2);
    }
    const char* baseA = (const char*)(Ag + m0 * args.lda);
    const char* baseB = (const char*)(Bg + n0);
    const int64_t stepA = (int64_t)BK * 2;
    const int64_t stepB = (int64_t)BK * args.ldb * 2;

    // the i-th slice of this wave (global slice index wave + i*NW) into ring slot s
    auto issue = [&](int i, int s) {
        const int kt = wave + i * NW;
        const char* a = baseA + kt * stepA;
        const char* b = baseB + kt * stepB;
        char* sa = obj(s) + wave * Cfg::SLOT;
        char* sb = sa + Cfg::A_BYTES;
#pragma unroll
        for (int j = 0; j < JA; ++j) direct_load16(a + offA_g[j], (lds_void_t*)(sa + j * 1024));
#pragma unroll
        for (int j = 0; j < JB; ++j) direct_load16(b + offB_g[j], (lds_void_t*)(sb + j * 1024));
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int g16 = lane >> 4, t16 = lane & 15;
    int offBj[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = j * 32 + 16 * (g16 & 1) + 4 * (t16 & 3);
        const int kr = 8 * (g16 >> 1) + (t16 >> 2);
        offBj[j] = kr * (2 * BN) + ((n >> 3) ^ swz_b<BCH>(kr)) * 16 + (n & 7) * 2;
    }
    struct Frags {
        u32x4 a[FM], b[FN];
    };
    auto read_frags = [&](Frags& f, int s, int step) {
        const char* sa = obj(s) + wave * Cfg::SLOT;
        const char* sb = sa + Cfg::A_BYTES;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = i * 32 + (lane & 31);
            const int c = (2 * step + (lane >> 5)) ^ swz_a<ACH>(row);
            f.a[i] = *(const lds_u32x4_t*)(sa + row * AROW + c * 16);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const i16x4 lo = lds_read_tr16(sb + offBj[j] + (16 * step) * (2 * BN));
            const i16x4 hi = lds_read_tr16(sb + offBj[j] + (16 * step + 4) * (2 * BN));
            f.b[j] = u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                           __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                           __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                           __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))};
        }
    };
    auto mfma_step = [&](const Frags& f) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<DT>(f.b[j], f.a[i], acc[i][j]);
    };

    // ---- this wave's K loop: private ring, no workgroup barrier ----------
    if (mine > 0) {
        constexpr int L = JA + JB;
        Frags F0, F1;
        const int pre = mine < RW ? mine : RW;
        for (int i = 0; i < pre; ++i) issue(i, i);
        if (pre == RW) wait_vmcnt<L * (RW - 1)>();
        else wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        read_frags(F0, 0, 0);
        for (int trip = 0; trip < mine; trip += RW) {
#pragma unroll
            for (int u = 0; u < RW; ++u) {
                const int i = trip + u;
                if (i >= mine) break;
#pragma unroll
                for (int s = 0; s < STEPS; ++s) {
                    Frags& cur = (s & 1) ? F1 : F0;
                    Frags& nxt = (s & 1) ? F0 : F1;
                    if (s + 1 < STEPS) {
                        read_frags(nxt, u, s + 1);
                    } else {
                        // own loads of slice i+1 complete; later ones stay in flight
                        if (i - 1 + RW <= mine - 1) wait_vmcnt<L * (RW - 2)>();
                        else wait_vmcnt<0>();
                        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slot u fully read
                        if (i + RW < mine) issue(i + RW, u);
                        if (i + 1 < mine) read_frags(nxt, (u + 1) % RW, 0);
                    }
                    mfma_step(cur);
                }
            }
        }
    }

    // ---- add the NW partial sums through LDS -------------------------------
    // Partial (wave w, MFMA tile q) goes to ring object q at offset w * 4 KB,
    // stored in the MFMA lane layout; wave w' then sums the tiles q with
    // q % NW == w' and writes them out.
    wait_vmcnt<0>();
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            char* dst = obj(i * FN + j) + wave * 4096 + lane * 16;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                *(float4*)(dst + r4 * 1024) =
                    float4{acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
        }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int q = i * FN + j;
            if (q % NW != wave) continue;
            float v[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) v[r] = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const char* src = obj(q) + w * 4096 + lane * 16;
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const float4 p = *(const float4*)(src + r4 * 1024);
                    v[4 * r4] += p.x;
                    v[4 * r4 + 1] += p.y;
                    v[4 * r4 + 2] += p.z;
                    v[4 * r4 + 3] += p.w;
                }
            }
            // accumulators hold C transposed (B is the first MFMA operand):
            // register 4q+t of lane l is C[l % 32][8q + 4 (l / 32) + t]
            const int64_t row = m0 + i * 32 + (lane & 31);
            const int64_t col0 = n0 + j * 32 + 4 * (lane >> 5);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int64_t col = col0 + 8 * q4;
                float x[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    x[t] = v[4 * q4 + t];
                    if constexpr (EPI) {
                        const float bt = (col + t < N) ? to_float<DT>(args.bias[col + t]) : 0.0f;
                        x[t] = x[t] + bt;
                        x[t] = (x[t] > 0.0f) ? x[t] : 0.0f;
                    }
                }
                const uint32_t lo = (uint32_t)from_float<DT>(x[0]) | ((uint32_t)from_float<DT>(x[1]) << 16);
                const uint32_t hi = (uint32_t)from_float<DT>(x[2]) | ((uint32_t)from_float<DT>(x[3]) << 16);
                if (row < M && col < N) store_out((u32x2*)(Cg + row * args.ldc + col), u32x2{lo, hi});
            }
        }
}

}  // namespace mg
