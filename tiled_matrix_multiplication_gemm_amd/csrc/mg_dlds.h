// Fast-path tile kernel for gfx950: both operands move global -> LDS with
// direct 16-byte loads (global_load_lds_dwordx4, no register staging), and the
// row-major B operand is read out of LDS with the transposing
// ds_read_b64_tr_b16, so no thread ever shuffles B in registers.
//
// One workgroup computes a BM x BN tile; the K loop streams BK-wide slices
// (BK = 32 or 64) through a ring of R LDS slots, so that up to R-2 slices are
// in flight while one feeds the matrix cores (the multi-stage pipeline of
// "Using Triton to optimise GEMM across chips", section 2.2, sized here by
// memory latency), with XOR-swizzled 16-byte chunks against bank conflicts
// (FlagOS cross-chip page, section 2.3).
//
// Preconditions (checked by the host): a tile's operand offsets fit in 31
// bits (BM * lda and 64 * ldb elements).  Rows past M and 8-element chunks
// past N are clamped to the last valid ones; what they feed are output rows
// and columns that are never stored.  K need not fill whole slices: in the
// last slice, 16-byte chunks (K-major operand) or k-rows (MN-major operand)
// that lie wholly past K take a load offset beyond the buffer resource's
// range, which the hardware answers with zeros, and when K % 8 != 0 the
// K-major fragments of that slice are masked in registers (the chunk that
// straddles K brings in elements of the row's padding).  Every 16-byte
// chunk that is loaded is 16-byte aligned and holds at least one element
// of the operand, so it lies in a page the operand occupies.
#pragma once

#include <type_traits>

#include "mg_tile.h"

namespace mg {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2_t;

// One 16-byte direct load per lane: global memory -> LDS at
// dst + 16 * lane (dst must be the same for the whole wave).
__device__ __forceinline__ void direct_load16(const void* src, lds_void_t* dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// Buffer resource over [base, base + 2^31) (word 3 = 0x00020000: untyped
// 32-bit data format, the gfx9 family's value; no swizzle, stride 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// The same direct load through a buffer resource: the per-lane part of the
// address is a 32-bit offset and the uniform part lives in scalar registers,
// so a load costs no vector address arithmetic (buffer_load_dwordx4 ... lds).
__device__ __forceinline__ void direct_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset, lds_void_t* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voffset, 0, 0, 0);
}

// Transposing LDS read: within each group of 16 lanes, lane t receives
// element t of each of the four 16-element rows that lanes 4r .. 4r+3 point at.
__device__ __forceinline__ i16x4 lds_read_tr16(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
}

template <int BM_, int BN_, int WM_, int WN_, int BK_ = 64, int R_ = 3, int PF_ = 1>
struct DldsCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int R = R_;                        // LDS slots in the ring (= slices in flight + 2)
    // LDS fragment reads run PF k16 steps ahead of the MFMAs (PF + 1 register
    // sets): a wave with few MFMAs per step needs more than one step of
    // them to cover the LDS latency
    static constexpr int PF = PF_;
    static constexpr int NW = WM * WN;                  // waves per workgroup
    static constexpr int NT = NW * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;  // output of one wave
    static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 MFMA tiles per wave
    static constexpr int STEPS = BK / 16;               // k16 MFMA steps per slice
    static constexpr int AROW = BK * 2;                 // bytes of one A row in LDS
    static constexpr int ACH = BK / 8;                  // 16-byte chunks per A row
    static constexpr int A_BYTES = BM * AROW;           // one slice of A
    static constexpr int B_BYTES = BK * BN * 2;         // one slice of B: BK k-rows of 2*BN bytes
    static constexpr int SLOT = A_BYTES + B_BYTES;
    static constexpr int JA = A_BYTES / 1024 / NW;      // 1 KB direct loads per wave per slice
    static constexpr int JB = B_BYTES / 1024 / NW;
    static constexpr int STAGES = R;
    static constexpr int LDS_BYTES = R * SLOT;
    static constexpr int BCH = BN / 8;                  // 16-byte chunks per B k-row
    // epilogue staging: each wave's output block passes through LDS (rows of
    // WTN bf16/fp16) so that the stores write whole 16-byte chunks of rows
    static constexpr int STAGE_BYTES = WTM * WTN * 2;
    static constexpr int STAGE_PER_SLOT = SLOT / STAGE_BYTES;
    static constexpr bool STAGED = STAGE_PER_SLOT >= 1 && STAGE_PER_SLOT * R >= NW &&
                                   (WTN / 8 == 4 || WTN / 8 == 8 || WTN / 8 == 16);
    static_assert(BK == 32 || BK == 64, "K slice must be 32 or 64");
    static_assert(R >= 3 && R <= 8, "ring of 3..8 slots");
    static_assert(PF >= 1 && PF < STEPS && STEPS % (PF + 1) == 0, "prefetch within a slice, register sets divide it");
    static_assert(JA * NW * 1024 == A_BYTES && JB * NW * 1024 == B_BYTES, "slice must split evenly over waves");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32x32");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KB of LDS per CU");
};

// Chunk swizzles, chosen so that the 16 lanes served per LDS cycle hit 16
// distinct 16-byte bank groups.  A: the MFMA operand read takes one chunk
// column of 32 consecutive rows (rows of 64 or 128 bytes).  B: k-rows are
// 2*BN bytes; a transposing read takes 32-byte pieces of 4 consecutive
// k-rows at the same columns.
template <int ACH>
__device__ __forceinline__ int swz_a(int row) {
    if constexpr (ACH == 8) return (row ^ (row >> 3)) & 7;
    else return (row >> 2) & 3;
}
// B: a transposing read takes 32 bytes from each of 4 consecutive k-rows;
// the swizzle puts those 4 pieces in 4 distinct 64-byte windows of the
// 256-byte bank row.  k-rows of 256 bytes or more all start a bank row, so
// the window is krow % 4; 128-byte k-rows alternate between the two halves
// of a bank row, so the window needs only (krow / 2) % 2.
template <int BCH>
__device__ __forceinline__ int swz_b(int krow) {
    static_assert(BCH >= 8, "k-rows of at least 128 bytes");
    if constexpr (BCH == 8) return 4 * ((krow >> 1) & 1);
    else return 4 * (krow & 3);
}

// The two operand layouts.  The MFMA wants, for each of 32 rows (of A) or
// columns (of B), 8 consecutive k values per lane.
//
// K-major (A as stored row-major [M,K]; B given transposed, [N,K]): E lines
// (rows of A or columns of B) whose K elements are contiguous, stored in LDS
// as E lines of BK*2 bytes with swizzled 16-byte chunks; a fragment is one
// ds_read_b128 of a chunk column over 32 lines.
//
// MN-major (B as stored row-major [K,N]; A given transposed, [K,M]): BK
// k-rows whose E elements are contiguous, stored as k-rows of E*2 bytes; a
// fragment is two transposing reads (ds_read_b64_tr_b16) per lane.
//
// Both give lane l the k values 16s + 8 (l / 32) + {0..7} of line l % 32 in
// the same order, so any pairing of the two layouts feeds the MFMA.  A slice
// is E*BK*2 bytes either way, loaded as 1 KB direct loads split over the NW
// waves.  K-major lines past the extent take an offset past the buffer
// resource's range, which the hardware answers with zeros without touching
// memory (the ragged last M-tile of an expert then streams only its real
// rows); MN-major 8-element chunks past it are clamped to the last valid
// chunk.
template <int E, int BK, int NW>
struct OpKM {
    static constexpr int CH = BK / 8, LINE = BK * 2, BYTES = E * LINE, J = BYTES / 1024 / NW;
    // byte offset (from the tile's first line of the slice) of load j of wave w, lane l
    // line of the tile and (swizzled) 16-byte chunk of the slice that load j
    // of wave w, lane l fetches
    __device__ static void load_pos(int w, int j, int lane, int& line, int& c) {
        const int q = w * J + j;
        line = q * (1024 / LINE) + lane / CH;
        c = (lane % CH) ^ swz_a<CH>(line);
    }
    __device__ static uint32_t load_off(int w, int j, int lane, int64_t e0, int64_t ext, int64_t ld) {
        int line, c;
        load_pos(w, j, lane, line, c);
        if (e0 + line >= ext) return 0x80000000u;
        return (uint32_t)(((int64_t)line * ld + 8 * c) * 2);
    }
    // first k (within the slice) of the chunk that load j of wave w, lane l fetches
    __device__ static int load_k(int w, int j, int lane) {
        int line, c;
        load_pos(w, j, lane, line, c);
        return 8 * c;
    }
    __device__ static const char* tile_base(const uint16_t* p, int64_t e0, int64_t ld) {
        return (const char*)(p + e0 * ld);
    }
    __device__ static int64_t slice_bytes(int64_t) { return (int64_t)BK * 2; }
    // per-lane LDS offset of 32-line block b of a wave whose lines start at woff
    __device__ static int frag_off(int woff, int b, int lane) { return (woff + b * 32 + (lane & 31)) * LINE; }
    __device__ static u32x4 read(const char* part, int off, int woff, int b, int s, int lane) {
        const int line = woff + b * 32 + (lane & 31);
        const int c = (2 * s + (lane >> 5)) ^ swz_a<CH>(line);
        return *(const lds_u32x4_t*)(part + off + c * 16);
    }
};

template <int E, int BK, int NW>
struct OpMN {
    static constexpr int CH = E / 8, LINE = E * 2, BYTES = BK * LINE, J = BYTES / 1024 / NW;
    // k-row (within the slice) that load j of wave w, lane l fetches from
    __device__ static int load_k(int w, int j, int lane) { return (w * J + j) * (512 / E) + (8 * lane) / E; }
    // chunks past the extent are clamped to the chunk that holds its last
    // element (e0 is a multiple of 8, so every chunk stays 16-byte aligned)
    __device__ static uint32_t load_off(int w, int j, int lane, int64_t e0, int64_t ext, int64_t ld) {
        const int krow = load_k(w, j, lane);
        const int c = (lane % CH) ^ swz_b<CH>(krow);
        const int64_t cn = (e0 + 8 * c < ext) ? 8 * c : ((ext - 1) & ~(int64_t)7) - e0;
        return (uint32_t)((krow * ld + cn) * 2);
    }
    __device__ static const char* tile_base(const uint16_t* p, int64_t e0, int64_t) { return (const char*)(p + e0); }
    __device__ static int64_t slice_bytes(int64_t ld) { return (int64_t)BK * ld * 2; }
    // lane l reads, through k-row 8 (g16 / 2) + t16 / 4, the piece of 4 lines
    // 16 (g16 % 2) + 4 (t16 % 4) .. of the block (g16, t16: lane's group of
    // 16 and index in it); the swizzle depends on the k-row modulo 4 only
    __device__ static int frag_off(int woff, int b, int lane) {
        const int g16 = lane >> 4, t16 = lane & 15;
        const int n = woff + b * 32 + 16 * (g16 & 1) + 4 * (t16 & 3);
        const int kr = 8 * (g16 >> 1) + (t16 >> 2);
        return kr * LINE + ((n >> 3) ^ swz_b<CH>(kr)) * 16 + (n & 7) * 2;
    }
    __device__ static u32x4 read(const char* part, int off, int, int, int s, int) {
        // k-rows 16s + {0..3} and 16s + {4..7} (+8 for the upper half-wave)
        const i16x4 lo = lds_read_tr16(part + off + (16 * s) * LINE);
        const i16x4 hi = lds_read_tr16(part + off + (16 * s + 4) * LINE);
        return u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                     __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                     __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                     __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))};
    }
};

// s_waitcnt vmcnt(N): wait until at most N vector memory operations of this
// wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for the LDS ring.  Unlike __syncthreads() it does not
// drain this wave's outstanding global->LDS loads (a release fence would
// wait for all of them, emptying the ring at every slice); each wave waits
// for exactly the loads it needs with wait_vmcnt before calling it.  Nor
// does it wait for this wave's LDS reads: the slot refilled after it is one
// whose reads every wave has already consumed (below).  The memory clobbers
// keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One LDS ring slot: a distinct shared-memory object per (slot index, kernel).
template <class Cfg, int DT, bool EPI, int MODE, bool TA, bool TB, bool KT>
struct DldsTag {};
template <int BYTES, int I, class Tag>
__device__ __forceinline__ char* lds_slot() {
    __shared__ __attribute__((aligned(1024))) char buf[BYTES];
    return buf;
}

// TA: A is given transposed (stored [K,M], lda = its k-row stride);
// TB: B is given transposed (stored [N,K], ldb = its row stride);
// KT: K is not a whole number of slices (this instance masks the last one;
// the others carry no trace of the masking).
template <class Cfg, int DT, bool EPI, int MODE, bool TA = false, bool TB = false, bool KT = false>
__global__ __launch_bounds__(Cfg::NT) void gemm_dlds_kernel(const KArgs args) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
    constexpr int FM = Cfg::FM, FN = Cfg::FN, JA = Cfg::JA, JB = Cfg::JB;
    constexpr int STEPS = Cfg::STEPS, R = Cfg::R;
    // R ring slots of [A slice | B slice], each its own LDS object so that the
    // compiler can tell reads of one slot from direct loads landing in another
    // (a single array would make it wait for every load in flight before each
    // LDS read).
    using Tag = DldsTag<Cfg, DT, EPI, MODE, TA, TB, KT>;
    using OA = std::conditional_t<TA, OpMN<Cfg::BM, Cfg::BK, Cfg::NW>, OpKM<Cfg::BM, Cfg::BK, Cfg::NW>>;
    using OB = std::conditional_t<TB, OpKM<Cfg::BN, Cfg::BK, Cfg::NW>, OpMN<Cfg::BN, Cfg::BK, Cfg::NW>>;
    static_assert(OA::J == Cfg::JA && OB::J == Cfg::JB, "operand slices split like the ring");
    auto slot_ptr = [&](int i) -> char* {  // i is a compile-time constant at every use
        switch (i) {
            case 0: return lds_slot<Cfg::SLOT, 0, Tag>();
            case 1: return lds_slot<Cfg::SLOT, 1, Tag>();
            case 2: if constexpr (R > 2) return lds_slot<Cfg::SLOT, 2, Tag>(); else return nullptr;
            case 3: if constexpr (R > 3) return lds_slot<Cfg::SLOT, 3, Tag>(); else return nullptr;
            case 4: if constexpr (R > 4) return lds_slot<Cfg::SLOT, 4, Tag>(); else return nullptr;
            case 5: if constexpr (R > 5) return lds_slot<Cfg::SLOT, 5, Tag>(); else return nullptr;
            case 6: if constexpr (R > 6) return lds_slot<Cfg::SLOT, 6, Tag>(); else return nullptr;
            default: if constexpr (R > 7) return lds_slot<Cfg::SLOT, 7, Tag>(); else return nullptr;
        }
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

    // ---- which tile (same order as the general kernel) --------------------
    const unsigned wg = tile_block<Cfg::NT>();
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
    int split = 0;  // split-K: which K range (workgroups of one split are contiguous)
    if constexpr (MODE == MODE_GROUPED) {
        int e, r0, rows;
        if (!grouped_tile<BM>(args, go, logical, e, r0, rows, pm, pn)) return;
        M = rows;
        Ag += (int64_t)r0 * args.lda;
        Bg += (int64_t)e * args.stride_we;
        Cg += (int64_t)r0 * args.ldc;
    } else {
        if constexpr (MODE == MODE_DENSE) batch_entry(args, logical, Ag, Bg, Cg);
        if constexpr (MODE == MODE_SPLITK) {
            const int per = args.tiles_m * args.tiles_n;
            split = logical / per;
            logical -= split * per;
        }
        grouped_order(logical, args.tiles_m, args.tiles_n, args.group_m, pm, pn);
    }
    const int64_t N = args.N, K = args.K;
    const int64_t m0 = (int64_t)pm * BM, n0 = (int64_t)pn * BN;
    int nk = (int)((K + BK - 1) / BK);
    int kt0 = 0;  // this workgroup's K slices are [kt0, kt0 + nk)
    if constexpr (MODE == MODE_SPLITK) {
        const int all = nk;
        kt0 = (int)((int64_t)split * all / args.splits);
        nk = (int)((int64_t)(split + 1) * all / args.splits) - kt0;
    }
    // Whether this workgroup's last slice reaches past K (its loads are then
    // masked), and whether a 16-byte chunk straddles K (K-major fragments of
    // that slice are then masked in registers).  A convolution's slices lie
    // within one kernel tap each, so its K is a whole number of slices.
    bool ragged = false, kmask = false;
    if constexpr (KT && MODE != MODE_CONV) {
        ragged = nk > 0 && (int64_t)(kt0 + nk) * BK > K;
        kmask = ragged && (K % 8) != 0;
    }

    // ---- per-lane source offsets of the direct loads ---------------------
    // 32-bit byte offsets from a workgroup-uniform base that advances by one
    // k-slice per step (the host guarantees they fit).  Load q = wave*J + j
    // of an operand fills bytes [q KB, q KB + 1 KB) of its part of the slot;
    // lane L lands at 16 L in it and fetches the logical chunk whose
    // swizzled position that is.
    uint32_t offA_g[JA];
#pragma unroll
    for (int j = 0; j < JA; ++j) offA_g[j] = OA::load_off(wave, j, lane, m0, M, args.lda);
    uint32_t offB_g[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) offB_g[j] = OB::load_off(wave, j, lane, n0, N, args.ldb);
    const int64_t stepA = OA::slice_bytes(args.lda);  // bytes per k-slice
    const int64_t stepB = OB::slice_bytes(args.ldb);
    const char* baseA = OA::tile_base(Ag, m0, args.lda) + kt0 * stepA;
    const char* baseB = OB::tile_base(Bg, n0, args.ldb) + kt0 * stepB;

    // Implicit-GEMM convolution: load j of this lane fetches, for output row
    // m (clamped to M-1 like any tile row) of image n at (oh, ow), the 16-byte
    // chunk `c` of the slice's channel run of input pixel (oh sh - ph + kh dh,
    // ow sw - pw + kw dw).  A slice lies within one kernel tap (C % BK == 0);
    // slices are issued in increasing order, so the tap (kh, kw) and channel
    // offset c0 advance by one slice per call.  Taps outside the image take
    // an offset past the buffer's range: the range check returns zeros.
    [[maybe_unused]] int32_t cv_ih0[JA], cv_iw0[JA];
    [[maybe_unused]] uint32_t cv_base[JA];
    [[maybe_unused]] int32_t cv_c0 = 0, cv_kw = 0, cv_khd = 0, cv_kwd = 0;
    if constexpr (MODE == MODE_CONV) {
        static_assert(!TA, "the gathered A operand is K-major");
        const ConvArgs& cv = args.conv;
        const uint32_t ohw = (uint32_t)cv.OH * (uint32_t)cv.OW;
#pragma unroll
        for (int j = 0; j < JA; ++j) {
            int line, c;
            OA::load_pos(wave, j, lane, line, c);
            const uint32_t m = (uint32_t)(m0 + line < M ? m0 + line : M - 1);  // M < 2^31
            const uint32_t n = m / ohw, rem = m - n * ohw;
            const uint32_t oh = rem / (uint32_t)cv.OW, ow = rem - oh * (uint32_t)cv.OW;
            cv_ih0[j] = (int32_t)oh * cv.sh - cv.ph;
            cv_iw0[j] = (int32_t)ow * cv.sw - cv.pw;
            // the host keeps the whole image batch below 2^31 bytes
            cv_base[j] = (n * (uint32_t)cv.H * (uint32_t)cv.W * (uint32_t)cv.C + 8u * (uint32_t)c) * 2u;
        }
    }

    // Prepacked A ([ceil(K/BKP), M, BKP], BKP = lda a multiple of BK): slice
    // kt is columns (kt % rp) BK .. of block kt / rp, whose rows are BKP
    // elements long.
    [[maybe_unused]] int rp = 1;
    if constexpr (MODE == MODE_PACKED_A) rp = (int)(args.lda / BK);

    // direct loads of k-slice kt into ring slot `slot` (a compile-time index)
    // (buffer resources rebased on the slice: offsets stay below 2^31);
    // `masked`: the slice reaches past K
    auto issue = [&](int kt, int slot, bool masked) {
        uint32_t offA[JA], offB[JB];
        __amdgpu_buffer_rsrc_t ra;
        if constexpr (MODE == MODE_CONV) {
            const ConvArgs& cv = args.conv;
            ra = buffer_rsrc((const char*)Ag);
#pragma unroll
            for (int j = 0; j < JA; ++j) {
                const int32_t ih = cv_ih0[j] + cv_khd, iw = cv_iw0[j] + cv_kwd;
                const bool in = (uint32_t)ih < (uint32_t)cv.H && (uint32_t)iw < (uint32_t)cv.W;
                offA[j] = in ? cv_base[j] + (((uint32_t)ih * (uint32_t)cv.W + (uint32_t)iw) * (uint32_t)cv.C +
                                             (uint32_t)cv_c0) * 2u
                             : 0x80000000u;
            }
            // next slice: the following channel run, else the next tap
            cv_c0 += BK;
            if (cv_c0 == cv.C) {
                cv_c0 = 0;
                cv_kwd += cv.dw;
                if (++cv_kw == cv.KW) {
                    cv_kw = 0;
                    cv_kwd = 0;
                    cv_khd += cv.dh;
                }
            }
        } else {
            if constexpr (MODE == MODE_PACKED_A) {
                const int kb = kt / rp, kr = kt - kb * rp;
                ra = buffer_rsrc((const char*)(Ag + ((int64_t)kb * M + m0) * args.lda + kr * BK));
            } else {
                ra = buffer_rsrc(baseA + kt * stepA);
            }
#pragma unroll
            for (int j = 0; j < JA; ++j) offA[j] = offA_g[j];
        }
#pragma unroll
        for (int j = 0; j < JB; ++j) offB[j] = offB_g[j];
        if constexpr (KT && MODE != MODE_CONV) {
            if (masked) {
                // chunks (K-major) or k-rows (MN-major) wholly past K: an
                // offset past the resource's range, answered with zeros
                const int64_t kbase = (int64_t)(kt0 + kt) * BK;
#pragma unroll
                for (int j = 0; j < JA; ++j)
                    if (kbase + OA::load_k(wave, j, lane) >= K) offA[j] = 0x80000000u;
#pragma unroll
                for (int j = 0; j < JB; ++j)
                    if (kbase + OB::load_k(wave, j, lane) >= K) offB[j] = 0x80000000u;
            }
        }
        const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(baseB + kt * stepB);
        char* sa = slot_ptr(slot);
        char* sb = sa + Cfg::A_BYTES;
#pragma unroll
        for (int j = 0; j < JA; ++j) direct_load16(ra, offA[j], (lds_void_t*)(sa + (wave * JA + j) * 1024));
#pragma unroll
        for (int j = 0; j < JB; ++j) direct_load16(rb, offB[j], (lds_void_t*)(sb + (wave * JB + j) * 1024));
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // ---- operand fragments ------------------------------------------------
    // Fragments of one k16 step: FM A fragments and FN B fragments (one
    // ds_read_b128 each if K-major, two transposing reads if MN-major).  Two
    // register sets alternate so that the reads of step s+1 are in flight
    // while the MFMAs of step s issue.
    int offAi[FM], offBj[FN];  // per-lane LDS offsets of the fragment blocks
#pragma unroll
    for (int i = 0; i < FM; ++i) offAi[i] = OA::frag_off(wm * Cfg::WTM, i, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) offBj[j] = OB::frag_off(wn * Cfg::WTN, j, lane);
    struct Frags {
        u32x4 a[FM], b[FN];
    };
    // `lv` is the number of this wave's 32-row MFMA blocks that hold output
    // rows below M (FM as a compile-time constant for full tiles): fragments
    // and MFMAs of the blocks past M are skipped.
    auto read_frags = [&](Frags& f, int slot, int s, auto lv) {
        const char* sa = slot_ptr(slot);
        const char* sb = sa + Cfg::A_BYTES;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            if (i >= lv) break;
            f.a[i] = OA::read(sa, offAi[i], wm * Cfg::WTM, i, s, lane);
        }
        if (lv == 0) return;
#pragma unroll
        for (int j = 0; j < FN; ++j) f.b[j] = OB::read(sb, offBj[j], wn * Cfg::WTN, j, s, lane);
    };
    // Slice t, step s: zero the elements at k >= K of the K-major fragments
    // (lane l holds k = 16 s + 8 (l / 32) + 0..7 of the slice) when a chunk
    // straddles K (K % 8 != 0); chunks wholly past K, and the MN-major
    // operand's k-rows past K, were loaded as zeros.
    auto mask_frags = [&](Frags& f, int t, int s) {
        const int64_t left = kmask ? K - ((int64_t)(kt0 + t) * BK + 16 * s) : 16;
        const int v0 = left <= 0 ? 0 : (left >= 16 ? 16 : (int)left);
        const int v = (lane >> 5) ? (v0 > 8 ? v0 - 8 : 0) : (v0 > 8 ? 8 : v0);
        auto keep = [&](u32x4& w) {
#pragma unroll
            for (int d = 0; d < 4; ++d) w[d] = (2 * d + 1 < v) ? w[d] : ((2 * d < v) ? (w[d] & 0xFFFFu) : 0u);
        };
        if constexpr (!TA) {
#pragma unroll
            for (int i = 0; i < FM; ++i) keep(f.a[i]);
        }
        if constexpr (TB) {
#pragma unroll
            for (int j = 0; j < FN; ++j) keep(f.b[j]);
        }
    };
    auto mfma_step = [&](const Frags& f, auto lv) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            if (i >= lv) break;
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<DT>(f.b[j], f.a[i], acc[i][j]);
        }
    };
    // Interleave the next step's LDS reads (FM + 2 FN instructions) with this
    // step's MFMAs (FM * FN instructions): two reads after each of the first
    // MFMAs, so that every read has several MFMAs' time to land before the
    // step ends.  Reads issued back to back in front of the MFMAs, or spread
    // to the end of the step, leave the matrix core idle.  In the step that
    // refills the ring, the NL direct loads are spread the same way, one per
    // MFMA: issued as one burst, they back up in the address unit and stall
    // the issuing waves.
    auto interleave = [&](auto nl) {
        constexpr int NL = decltype(nl)::value;
        constexpr int NR = FM + 2 * FN, Q = FM * FN;
        constexpr int PAIRS = (NR + 1) / 2 < Q ? (NR + 1) / 2 : Q;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            if (q < PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two DS reads
            if (q < NL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one direct load
        }
        if constexpr (NR > 2 * PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, NR - 2 * PAIRS, 0);
        if constexpr (NL > Q) __builtin_amdgcn_sched_group_barrier(0x020, NL - Q, 0);
    };

    // ---- main loop over k-slices -------------------------------------------
    // Ring of R LDS slots; slice t lives in slot t % R.  The fragments of
    // k16 step g are read PF steps before its MFMAs, into register set
    // g % (PF + 1).  Reading the first step of slice t+1 (at step STEPS - PF
    // of slice t) needs slice t+1 in LDS everywhere: there the wave waits for
    // its own loads of slice t+1, the workgroup synchronises, and slice
    // t+R-1 is issued into the slot of slice t-1.  Every read of slice t-1
    // fed an MFMA of slice t-1 before this barrier, so no wave needs to drain
    // its LDS reads at the barrier.  Up to R-2 slices are in flight while one
    // is consumed.
    //
    // Trips of R slices (slice trip + u in slot u, u a compile-time index).
    // While every slice of a trip still has a slice t + R - 1 to issue, the
    // trip is one straight-line block with constant waits, which lets the
    // scheduler interleave reads and MFMAs across the slice boundary; the
    // last trips take the general form with run-time conditions.
    constexpr int L = JA + JB;  // loads per wave per slice
    constexpr int PF = Cfg::PF, NF = PF + 1;
    Frags F[NF];
    auto slice = [&](const int t, const int u, const bool steady, auto lv) {
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            Frags& cur = F[s % NF];
            Frags& nxt = F[(s + PF) % NF];
            if (s + PF < STEPS) {
                read_frags(nxt, u, s + PF, lv);
            } else if (steady) {
                if (s + PF == STEPS) {
                    wait_vmcnt<L * (R - 3)>();
                    ring_barrier();
                    issue(t + R - 1, (u + R - 1) % R, false);
                }
                read_frags(nxt, (u + 1) % R, s + PF - STEPS, lv);
            } else {
                if (s + PF == STEPS) {
                    // slices issued so far: 0 .. min(t+R-2, nk-1); in steady
                    // state the R-3 slices after t+1 stay in flight, near the
                    // end wait for all
                    if (t + R - 2 <= nk - 1) wait_vmcnt<L * (R - 3)>();
                    else wait_vmcnt<0>();
                    ring_barrier();
                    if (t + R - 1 < nk) issue(t + R - 1, (u + R - 1) % R, ragged && t + R - 1 == nk - 1);
                }
                if (t + 1 < nk) read_frags(nxt, (u + 1) % R, s + PF - STEPS, lv);
            }
            // K-tail instance: outside the steady trips every step masks its
            // K-major fragments with selects (no branch, so the step stays one
            // block in which reads and MFMAs interleave); only the last slice
            // has anything to clear
            if constexpr (KT) {
                if (!steady) mask_frags(cur, t, s);
            }
            mfma_step(cur, lv);
            if (steady && s + PF == STEPS) interleave(std::integral_constant<int, JA + JB>{});
            else interleave(std::integral_constant<int, 0>{});
        }
    };
    auto main_loop = [&](auto lv) {
        if (nk <= 0) return;
        const int pre = nk < R - 1 ? nk : R - 1;
        for (int t = 0; t < pre; ++t) issue(t, t, ragged && t == nk - 1);
        if (pre == R - 1) wait_vmcnt<L * (R - 2)>();  // slice 0 landed, R-2 slices still in flight
        else wait_vmcnt<0>();
        ring_barrier();
#pragma unroll
        for (int p = 0; p < PF; ++p) read_frags(F[p], 0, p, lv);
        int trip = 0;
        // steady trips: slices trip .. trip+R-1 all satisfy t + R - 1 < nk;
        // a last slice that reaches past K is issued and consumed outside them
        const int nk_steady = ragged ? nk - 1 : nk;
        for (; trip + 2 * R - 1 <= nk_steady; trip += R) {
#pragma unroll
            for (int u = 0; u < R; ++u) slice(trip + u, u, true, lv);
        }
        for (; trip < nk; trip += R) {
#pragma unroll
            for (int u = 0; u < R; ++u) {
                if (trip + u >= nk) break;
                slice(trip + u, u, false, lv);
            }
        }
    };
    // Waves whose rows all lie below M run the loop with every MFMA; the
    // others (edge tiles, the ragged last tile of an expert) skip the 32-row
    // blocks past M.  Both forms take the same barriers in the same order, and
    // the choice is made on a scalar (wave-uniform) value.
    const int64_t wave_rows = M - m0 - wm * Cfg::WTM;
    const int live = __builtin_amdgcn_readfirstlane(
        (int)(wave_rows >= Cfg::WTM ? FM : (wave_rows <= 0 ? 0 : (wave_rows + 31) / 32)));
    // Fused epilogue: the bias values of this lane's output columns are
    // loaded before the K loop, so their latency is not paid at the end.
    // Lane l's columns in block j are, for group q, the 4 adjacent columns
    // j*32 + 4 (l / 32) + 8 q: one 8-byte load each when the bias is 8-byte
    // aligned (element by element for the group that straddles N); otherwise
    // the epilogue reads the bias element by element.  Loads older than the
    // ring's only make its waits stricter.  A wave whose accumulators take
    // 256 registers has none to spare for the bias (they would spill), so
    // it reads the bias in the epilogue.
    constexpr bool kBiasInRegs = FM * FN * 16 < 256;
    [[maybe_unused]] u32x2 bias_v[FN][4];
    [[maybe_unused]] bool bias_pre = false;
    if constexpr (EPI && kBiasInRegs) {
        bias_pre = ((uintptr_t)args.bias & 7) == 0;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t col = n0 + wn * Cfg::WTN + j * 32 + 4 * (lane >> 5) + 8 * q;
                if (bias_pre && col + 4 <= N) {
                    bias_v[j][q] = *(const u32x2*)(args.bias + col);
                } else {
                    uint32_t h[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) h[t] = (bias_pre && col + t < N) ? (uint32_t)args.bias[col + t] : 0u;
                    bias_v[j][q] = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
                }
            }
    }
    if (live == FM) main_loop(std::integral_constant<int, FM>{});
    else main_loop(live);

    // ---- epilogue: (bias, ReLU), one rounding, stores -------------------
    // The MFMAs take B as their first operand, so each accumulator tile holds
    // C transposed: register r of lane l is C[l % 32][8 (r / 4) + 4 (l / 32)
    // + r % 4] of the 32x32 tile, i.e. a lane owns 4 adjacent columns of one
    // row per group of 4 registers.  Those 8 bytes go to LDS (the ring is free
    // once every wave has left the K loop), row-major per wave with XOR-
    // swizzled 16-byte chunks; the wave then reads back whole chunks and
    // writes each output row as contiguous 16-byte pieces, 8 rows per store
    // (the one chunk of a row that straddles N, when N % 8 != 0, element by
    // element).
    // One 32x32 tile at a time (a scheduling barrier keeps the compiler from
    // pulling every accumulator out at once); interior tiles skip the checks.
    const bool interior = (m0 + BM <= M) && (n0 + BN <= N);
    auto pack4 = [&](const f32x16& c, int j, int q, int64_t col) -> u32x2 {
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            v[t] = c[4 * q + t];
            if constexpr (EPI) {
                float bt;
                if (kBiasInRegs && bias_pre) bt = to_float<DT>((uint16_t)(bias_v[j][q][t >> 1] >> (16 * (t & 1))));
                else bt = (col + t < N) ? to_float<DT>(args.bias[col + t]) : 0.0f;
                v[t] = v[t] + bt;
                v[t] = (v[t] > 0.0f) ? v[t] : 0.0f;
            }
        }
        return u32x2{(uint32_t)from_float<DT>(v[0]) | ((uint32_t)from_float<DT>(v[1]) << 16),
                     (uint32_t)from_float<DT>(v[2]) | ((uint32_t)from_float<DT>(v[3]) << 16)};
    };
    if constexpr (MODE == MODE_SPLITK) {
        // fp32 partial tile of this split: 4 adjacent columns per lane and
        // register group, one 16-byte store each
        float* W = args.ws + (int64_t)split * M * N;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t row = m0 + wm * Cfg::WTM + i * 32 + (lane & 31);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                const int64_t col0 = n0 + wn * Cfg::WTN + j * 32 + 4 * (lane >> 5);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t col = col0 + 8 * q;
                    const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    if (row < M && col < N) *(f32x4*)(W + row * N + col) = v;
                }
            }
        }
    } else if constexpr (Cfg::STAGED) {
        constexpr int CH = Cfg::WTN / 8;  // 16-byte chunks per staged row
        constexpr int RB = Cfg::WTN * 2;  // bytes per staged row
        auto stage_swz = [](int row) { return (row ^ (row >> 3)) & (CH - 1); };
        // A ds_write_b64 is served 16 lanes at a time over 128 bytes of
        // banks (what the bank-conflict counter shows): rows 0..15 of a block,
        // all at the same 8-byte half of their chunks.  The chunk swizzle
        // separates them except for pairs of rows that differ in bit
        // HS = log2(CH) (alone for CH = 4, together with bit 0 for CH = 8),
        // so swapping the halves of the rows whose bit HS is set puts all 16
        // in distinct banks.  (Bit 4 for CH = 8 left a two-way conflict on
        // every write.)
        // The read-back swaps them back.
        constexpr int HS = CH == 4 ? 2 : 3;
        auto stage_half = [](int row) { return (row >> HS) & 1; };
        wait_vmcnt<0>();
        ring_barrier();  // every wave is out of the K loop: the ring is free
        char* stage = nullptr;
#pragma unroll
        for (int u = 0; u < R; ++u)
            if (wave / Cfg::STAGE_PER_SLOT == u) stage = slot_ptr(u) + (wave % Cfg::STAGE_PER_SLOT) * Cfg::STAGE_BYTES;
        // 32-row blocks wholly past M (edge tiles, an expert's ragged last
        // tile) are neither staged nor read back: nothing of them is stored
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            if (i >= live) break;
            const int row = i * 32 + (lane & 31);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                const int cl = j * 32 + 4 * (lane >> 5);  // first column of this lane's group, q = 0
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = cl + 8 * q;
                    const u32x2 w = pack4(acc[i][j], j, q, n0 + wn * Cfg::WTN + c);
                    *(lds_u32x2_t*)(stage + row * RB + ((c >> 3) ^ stage_swz(row)) * 16 +
                                    (((c & 7) * 2) ^ (8 * stage_half(row)))) = w;
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // own writes done before reading them back
        constexpr int ROWS_PER_LOAD = 64 / CH;
        const int rsub = lane / CH, ch = lane % CH;
        const int64_t col = n0 + wn * Cfg::WTN + ch * 8;
#pragma unroll
        for (int it = 0; it < Cfg::WTM / ROWS_PER_LOAD; ++it) {
            if (it * ROWS_PER_LOAD >= live * 32) break;
            const int row = it * ROWS_PER_LOAD + rsub;
            u32x4 w = *(const lds_u32x4_t*)(stage + row * RB + (ch ^ stage_swz(row)) * 16);
            if (stage_half(row)) w = u32x4{w[2], w[3], w[0], w[1]};
            const int64_t grow = m0 + wm * Cfg::WTM + row;
            if (interior || (grow < M && col + 8 <= N)) {
                store_out((u32x4*)(Cg + grow * args.ldc + col), w);
            } else if (grow < M && col < N) {
                // the chunk that straddles N (N % 8 != 0): its valid elements
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (col + e < N) Cg[grow * args.ldc + col + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t row = m0 + wm * Cfg::WTM + i * 32 + (lane & 31);
            const bool row_ok = interior || row < M;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                const int64_t col0 = n0 + wn * Cfg::WTN + j * 32 + 4 * (lane >> 5);
                uint16_t* cp = Cg + row * args.ldc + col0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x2 w = pack4(acc[i][j], j, q, col0 + 8 * q);
                    if (row_ok && (interior || col0 + 8 * q + 4 <= N)) {
                        store_out((u32x2*)(cp + 8 * q), w);
                    } else if (row_ok) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (col0 + 8 * q + e < N) cp[8 * q + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                    }
                }
            }
        }
    }
}

// Split-K reduction: C = sum over splits of the fp32 partials, in split
// order (deterministic), one rounding; 8 adjacent outputs per thread
// (N % 8 == 0 on this path), 16-byte loads and stores.
template <int DT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* ws, uint16_t* C, int64_t M, int64_t N,
                                                            int64_t ldc, int splits) {
    const int64_t groups = M * (N / 8);
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups; g += (int64_t)gridDim.x * 256) {
        const int64_t row = g / (N / 8), col = (g % (N / 8)) * 8;
        f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < splits; ++s) {
            const float* p = ws + (int64_t)s * M * N + row * N + col;
            lo += *(const f32x4*)p;
            hi += *(const f32x4*)(p + 4);
        }
        u32x4 o;
        o[0] = (uint32_t)from_float<DT>(lo[0]) | ((uint32_t)from_float<DT>(lo[1]) << 16);
        o[1] = (uint32_t)from_float<DT>(lo[2]) | ((uint32_t)from_float<DT>(lo[3]) << 16);
        o[2] = (uint32_t)from_float<DT>(hi[0]) | ((uint32_t)from_float<DT>(hi[1]) << 16);
        o[3] = (uint32_t)from_float<DT>(hi[2]) | ((uint32_t)from_float<DT>(hi[3]) << 16);
        store_out((u32x4*)(C + row * ldc + col), o);
    }
}

}  // namespace mg
