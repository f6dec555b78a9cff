// The table of compiled tile shapes, shared by the host code and the
// per-row translation units that instantiate the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

#include "mi355gemm.h"
#include "mg_tile.h"
#include "mg_dlds.h"
#include "mg_kslab.h"

namespace mg {

// ---- configuration table ---------------------------------------------------
// One row per compiled tile shape.  The table is static: rows are chosen by
// shape class in select_config(), which an offline sweep tunes; there is no
// run-time search.
// Each row has a general kernel (register-staged loads, any K and N) and,
// all but row 5, a direct-to-LDS fast kernel that takes any K and N as well
// (K tails in the separate tail instances).  The general kernel runs only on
// row 5 and where a tile's operand span does not fit the fast kernel's
// 31-bit load offsets (leading dimensions of millions of elements).
using Cfg0 = TileCfg<256, 256, 64, 2, 4>;  // large square problems, eight waves (two per SIMD)
using Cfg1 = TileCfg<128, 128, 64, 2, 2>;  // mid-size, grouped
using Cfg2 = TileCfg<64, 64, 64, 2, 2>;    // small problems: enough tiles to fill 256 CUs
using Cfg3 = TileCfg<128, 256, 64, 2, 2>;
using Cfg4 = TileCfg<256, 128, 64, 2, 2>;
using Cfg5 = TileCfg<128, 128, 32, 2, 2>;
using Cfg6 = TileCfg<256, 256, 64, 2, 4>;  // general fallback keeps eight waves
// fast kernels: <BM, BN, waves M, waves N, K slice, LDS ring slots, fragment prefetch in
// k16 steps>: rows whose waves issue few MFMAs per step read their fragments
// three steps ahead (1024 x 1024 x 2048: 0.0089 -> 0.0085 ms)
using Fast0 = DldsCfg<256, 256, 2, 4, 32, 5>;
// two workgroups per CU (K slices of 32 in a ring of 5 at 80 KB): the
// slices of 64 in a ring of 3 (96 KB, one workgroup per CU) lost to the
// 256 x 64 row everywhere; this form beats it by 2-8 % on mid-size outputs
using Fast1 = DldsCfg<128, 128, 2, 2, 32, 5, 1>;
// a ring of 5 at 80 KB, so that two workgroups share a CU wherever there are
// more tiles than CUs (one more slot bought nothing, and cost the second
// workgroup: 1000^3 0.0124 -> 0.0105 ms, a 14 x 14 x 256 convolution layer
// 0.0203 -> 0.0146 ms, 1024 x 1024 x 2048 unchanged)
using Fast2 = DldsCfg<64, 64, 2, 2, 64, 5, 3>;
using Fast3 = DldsCfg<128, 256, 2, 2, 32, 4>;
// two workgroups per CU (eight waves of 64 x 64, 118-122 registers, a ring of
// 3 at 72 KB): one workgroup's epilogue runs beside the other's K loop, which
// pays where storing the output dominates (attention scores: 0.347 -> 0.277 ms)
using Fast4 = DldsCfg<256, 128, 4, 2, 32, 3>;
using Fast6 = DldsCfg<256, 256, 2, 2, 32, 5>;
using Cfg7 = TileCfg<64, 64, 64, 2, 2>;
using Fast7 = SlabCfg<64, 64, 4, 32, 4>;  // K split over the 4 waves of the workgroup
// tall, thin outputs (N of 64 or 128 and many rows: convolution GEMMs, narrow
// projections): a whole 64-column slab per tile, eight waves of 64 x 32
using Cfg8 = TileCfg<256, 64, 64, 4, 2>;
using Fast8 = DldsCfg<256, 64, 4, 2, 64, 4, 3>;
// the same slab two workgroups per CU (four waves of 64 x 64, 70 + 64
// registers, a ring of 4 at 80 KB): where K is short the tile is mostly
// ring fill and epilogue, and the other workgroup's K loop runs beside
// them (the 3x3 convolution: 0.0187 -> 0.0149 ms)
using Cfg9 = TileCfg<256, 64, 64, 4, 2>;
using Fast9 = DldsCfg<256, 64, 4, 1, 32, 4, 1>;

inline constexpr int kNumConfigs = 10;

// Kernel family of the last launch (mg_last_kernel): 0 general, 1 direct-to-LDS, 2 K-split.
void note_kernel(int family);
// GROUP_M of the tile order (the Gluon matmul example's grouping; "Triton
// study notes" suggest 8): 4 measured 0.3-1.0 % faster than 8 on eight
// large shapes and 0.6-1.6 % in three power-capped 8192^3 soaks.
inline constexpr int kGroupM = 4;

template <class F>
struct is_slab : std::false_type {};
template <int BM, int BN, int NW, int BK, int RW>
struct is_slab<SlabCfg<BM, BN, NW, BK, RW>> : std::true_type {};

// Launch row `cfg` (0 .. kNumConfigs-1) on stream s; ta / tb: A / B given
// transposed.  Defined one per row in mg_row<cfg>.hip so that the rows
// compile in parallel.
#define MG_DECLARE_ROW(n)                                                                                   \
    mg_status launch_row##n(int dt, bool epi, int mode, int ta, int tb, const KArgs& a, int64_t grid,     \
                            hipStream_t s)
MG_DECLARE_ROW(0);
MG_DECLARE_ROW(1);
MG_DECLARE_ROW(2);
MG_DECLARE_ROW(3);
MG_DECLARE_ROW(4);
MG_DECLARE_ROW(5);
MG_DECLARE_ROW(6);
MG_DECLARE_ROW(7);
MG_DECLARE_ROW(8);
MG_DECLARE_ROW(9);

// The same for problems whose K is not a whole number of the row's slices
// (direct-to-LDS kernel instances that mask the last slice), defined in
// mg_row<cfg>_tail.hip; rows without such a kernel define it as an error.
#define MG_DECLARE_ROW_TAIL(n)                                                                              \
    mg_status launch_row##n##_tail(int dt, bool epi, int mode, int ta, int tb, const KArgs& a, int64_t grid, \
                                   hipStream_t s)
MG_DECLARE_ROW_TAIL(0);
MG_DECLARE_ROW_TAIL(1);
MG_DECLARE_ROW_TAIL(2);
MG_DECLARE_ROW_TAIL(3);
MG_DECLARE_ROW_TAIL(4);
MG_DECLARE_ROW_TAIL(5);
MG_DECLARE_ROW_TAIL(6);
MG_DECLARE_ROW_TAIL(7);
MG_DECLARE_ROW_TAIL(8);
MG_DECLARE_ROW_TAIL(9);
using RowLauncher = mg_status (*)(int, bool, int, int, int, const KArgs&, int64_t, hipStream_t);

// fp32 GEMM: one configuration (mg_f32.h), defined in mg_f32.hip
// fp32 kernel tiles: 0 = 128 x 128 (large outputs), 1 = 64 x 64 (outputs
// that leave the CUs idle at 128 x 128).  K slices of 16 values.
inline constexpr int kF32NumTiles = 2, kF32SliceK = 16;
inline constexpr int kF32TileM[kF32NumTiles] = {128, 64}, kF32TileN[kF32NumTiles] = {128, 64};
mg_status launch_f32(int tile, bool epi, const KArgs& a, int64_t grid, hipStream_t s);

}  // namespace mg
