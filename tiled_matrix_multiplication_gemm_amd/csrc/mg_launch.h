// Kernel launchers: pick the direct-to-LDS, K-split or general kernel of a
// table row for the problem and launch it.  Included by the per-row
// translation units only.
#pragma once

#include "mg_table.h"

namespace mg {

template <class C, int DT, bool EPI, int MODE>
mg_status launch_cfg(const KArgs& a, int64_t grid, hipStream_t stream) {
    (void)hipGetLastError();  // clear a stale error so the check below is ours
    hipLaunchKernelGGL((gemm_tile_kernel<C, DT, EPI, MODE>), tile_grid(grid, C::NT), dim3(C::NT), 0, stream, a);
    return hipGetLastError() == hipSuccess ? MG_OK : MG_ERR_HIP;
}

template <class F, int DT, bool EPI, int MODE, bool TA = false, bool TB = false, bool KT = false>
mg_status launch_fast(const KArgs& a, int64_t grid, hipStream_t stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((gemm_dlds_kernel<F, DT, EPI, MODE, TA, TB, KT>), tile_grid(grid, F::NT), dim3(F::NT), 0, stream,
                       a);
    return hipGetLastError() == hipSuccess ? MG_OK : MG_ERR_HIP;
}

// dense GEMM on the direct-to-LDS kernel with A and/or B given transposed
template <class F, int DT, bool EPI, bool KT>
mg_status launch_fast_t(int ta, int tb, const KArgs& a, int64_t grid, hipStream_t s) {
    if (ta && tb) return launch_fast<F, DT, EPI, MODE_DENSE, true, true, KT>(a, grid, s);
    if (ta) return launch_fast<F, DT, EPI, MODE_DENSE, true, false, KT>(a, grid, s);
    if (tb) return launch_fast<F, DT, EPI, MODE_DENSE, false, true, KT>(a, grid, s);
    return launch_fast<F, DT, EPI, MODE_DENSE, false, false, KT>(a, grid, s);
}

template <class C, int DT>
mg_status launch_general(bool epi, int mode, const KArgs& a, int64_t grid, hipStream_t s) {
    if (mode == MODE_GROUPED) return launch_cfg<C, DT, false, MODE_GROUPED>(a, grid, s);
    if (mode == MODE_PACKED_A) return launch_cfg<C, DT, false, MODE_PACKED_A>(a, grid, s);
    return epi ? launch_cfg<C, DT, true, MODE_DENSE>(a, grid, s) : launch_cfg<C, DT, false, MODE_DENSE>(a, grid, s);
}

template <class F, int DT, bool EPI>
mg_status launch_slab(const KArgs& a, int64_t grid, hipStream_t stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((gemm_kslab_kernel<F, DT, EPI>), tile_grid(grid, F::NT), dim3(F::NT), 0, stream, a);
    return hipGetLastError() == hipSuccess ? MG_OK : MG_ERR_HIP;
}

// split-K: partial products of every split into the workspace, then their
// sum in split order into C (both on stream s)
template <class F, int DT, bool KT>
mg_status launch_split(int ta, int tb, const KArgs& a, int64_t grid, hipStream_t s) {
    mg_status st;
    if (ta && tb) st = launch_fast<F, DT, false, MODE_SPLITK, true, true, KT>(a, grid, s);
    else if (ta) st = launch_fast<F, DT, false, MODE_SPLITK, true, false, KT>(a, grid, s);
    else if (tb) st = launch_fast<F, DT, false, MODE_SPLITK, false, true, KT>(a, grid, s);
    else st = launch_fast<F, DT, false, MODE_SPLITK, false, false, KT>(a, grid, s);
    if (st != MG_OK) return st;
    const int64_t groups = a.M * (a.N / 8);
    const int64_t blocks = (groups + 255) / 256 < 8192 ? (groups + 255) / 256 : 8192;
    hipLaunchKernelGGL((splitk_reduce_kernel<DT>), dim3((unsigned)blocks), dim3(256), 0, s, (const float*)a.ws, a.C,
                       a.M, a.N, a.ldc, a.splits);
    return hipGetLastError() == hipSuccess ? MG_OK : MG_ERR_HIP;
}

// KT: K is not a whole number of the kernel's slices (the instance that
// masks the last slice; the others carry no trace of it)
template <class F, int DT, bool KT>
mg_status launch_direct(bool epi, int mode, int ta, int tb, const KArgs& a, int64_t grid, hipStream_t s) {
    if constexpr (is_slab<F>::value) {
        (void)mode, (void)ta, (void)tb;
        if constexpr (KT) return MG_ERR_BAD_CONFIG;
        else return epi ? launch_slab<F, DT, true>(a, grid, s) : launch_slab<F, DT, false>(a, grid, s);
    } else {
        if (mode == MODE_SPLITK) return launch_split<F, DT, KT>(ta, tb, a, grid, s);
        if (mode == MODE_GROUPED) return launch_fast<F, DT, false, MODE_GROUPED, false, false, KT>(a, grid, s);
        if (mode == MODE_PACKED_A) return launch_fast<F, DT, false, MODE_PACKED_A, false, false, KT>(a, grid, s);
        if (mode == MODE_CONV) {
            if constexpr (KT) {
                return MG_ERR_BAD_CONFIG;  // a convolution's K is a whole number of slices
            } else {
                if (epi) return tb ? launch_fast<F, DT, true, MODE_CONV, false, true>(a, grid, s)
                                   : launch_fast<F, DT, true, MODE_CONV, false, false>(a, grid, s);
                return tb ? launch_fast<F, DT, false, MODE_CONV, false, true>(a, grid, s)
                          : launch_fast<F, DT, false, MODE_CONV, false, false>(a, grid, s);
            }
        }
        return epi ? launch_fast_t<F, DT, true, KT>(ta, tb, a, grid, s)
                   : launch_fast_t<F, DT, false, KT>(ta, tb, a, grid, s);
    }
}

// The K-tail instances of row F (defined in their own translation unit, so
// that the two halves of a row compile in parallel).
template <class F>
mg_status launch_direct_tail(int dt, bool epi, int mode, int ta, int tb, const KArgs& a, int64_t grid, hipStream_t s) {
    if constexpr (std::is_void<F>::value || is_slab<F>::value) {
        return MG_ERR_BAD_CONFIG;
    } else {
        return dt == DT_F16 ? launch_direct<F, DT_F16, true>(epi, mode, ta, tb, a, grid, s)
                            : launch_direct<F, DT_BF16, true>(epi, mode, ta, tb, a, grid, s);
    }
}

// Whether the direct-to-LDS kernel of row F takes this problem: every
// per-tile operand offset within 31 bits (K-major operand: a tile's lines;
// MN-major: a slice's k-rows).  The direct-to-LDS kernel takes any K and N;
// split-K needs N in whole 8-element chunks (its fp32 partials are stored
// and summed 8 columns at a time), a convolution slices that lie within one
// kernel tap, a prepacked A blocks of whole slices.  The K-split kernel
// takes dense row-major problems with K in whole slices and N % 8 == 0.
template <class F>
bool direct_fits(int mode, int ta, int tb, const KArgs& a) {
    constexpr int64_t LIM = (int64_t)1 << 31;
    if (is_slab<F>::value) {
        if (mode != MODE_DENSE || ta || tb) return false;
        if (a.K % F::BK != 0 || a.N % 8 != 0) return false;
    }
    if (mode == MODE_SPLITK && a.N % 8 != 0) return false;
    if (mode == MODE_PACKED_A && (ta || tb || a.lda % F::BK != 0)) return false;
    if (mode == MODE_CONV && (ta || a.conv.C % F::BK != 0)) return false;  // a slice within one kernel tap
    const int64_t a_span = ta ? 64 * a.lda * 2 : (int64_t)F::BM * a.lda * 2;
    const int64_t b_span = tb ? (int64_t)F::BN * a.ldb * 2 : 64 * a.ldb * 2;
    return a_span < LIM && b_span < LIM;
}

// F = void: the row has no direct-to-LDS kernel.  Transposed operands exist
// on the direct-to-LDS kernel only.
template <class C, class F>
mg_status launch_dt(int dt, bool epi, int mode, int ta, int tb, const KArgs& a, int64_t grid, hipStream_t s,
                    RowLauncher tail) {
    if constexpr (!std::is_void<F>::value) {
        if (direct_fits<F>(mode, ta, tb, a)) {
            if (a.dry) return MG_OK;
            mg_status st;
            if (!is_slab<F>::value && a.K % F::BK != 0)
                st = tail(dt, epi, mode, ta, tb, a, grid, s);
            else
                st = dt == DT_F16 ? launch_direct<F, DT_F16, false>(epi, mode, ta, tb, a, grid, s)
                                  : launch_direct<F, DT_BF16, false>(epi, mode, ta, tb, a, grid, s);
            if (st == MG_OK) note_kernel(is_slab<F>::value ? 2 : 1);
            return st;
        }
    }
    if (ta || tb || mode == MODE_SPLITK || mode == MODE_CONV) return MG_ERR_UNSUPPORTED_LAYOUT;
    if (a.dry) return MG_OK;
    const mg_status st = dt == DT_F16 ? launch_general<C, DT_F16>(epi, mode, a, grid, s)
                                      : launch_general<C, DT_BF16>(epi, mode, a, grid, s);
    if (st == MG_OK) note_kernel(0);
    return st;
}

}  // namespace mg

#define MG_DEFINE_ROW(n, C, F)                                                                      \
    namespace mg {                                                                                  \
    MG_DECLARE_ROW(n) { return launch_dt<C, F>(dt, epi, mode, ta, tb, a, grid, s, &launch_row##n##_tail); } \
    }

#define MG_DEFINE_ROW_TAIL(n, F)                                                                    \
    namespace mg {                                                                                  \
    MG_DECLARE_ROW_TAIL(n) { return launch_direct_tail<F>(dt, epi, mode, ta, tb, a, grid, s); }    \
    }
