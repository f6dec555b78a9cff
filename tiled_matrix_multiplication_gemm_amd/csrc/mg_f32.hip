// fp32 GEMM kernel (mg_f32.h) and its launcher.
#include "mg_table.h"
#include "mg_f32.h"

namespace mg {

using CfgF32L = F32Cfg<kF32TileM[0], kF32TileN[0], 2, 2, kF32SliceK, 4>;
using CfgF32S = F32Cfg<kF32TileM[1], kF32TileN[1], 2, 2, kF32SliceK, 6>;

template <class Cfg>
static void launch_cfg_f32(bool epi, const KArgs& a, int64_t grid, hipStream_t s) {
    if (epi)
        hipLaunchKernelGGL((gemm_f32_kernel<Cfg, true>), tile_grid(grid, Cfg::NT), dim3(Cfg::NT), 0, s, a);
    else
        hipLaunchKernelGGL((gemm_f32_kernel<Cfg, false>), tile_grid(grid, Cfg::NT), dim3(Cfg::NT), 0, s, a);
}

mg_status launch_f32(int tile, bool epi, const KArgs& a, int64_t grid, hipStream_t s) {
    (void)hipGetLastError();
    switch (tile) {
        case 0: launch_cfg_f32<CfgF32L>(epi, a, grid, s); break;
        case 1: launch_cfg_f32<CfgF32S>(epi, a, grid, s); break;
        default: return MG_ERR_BAD_CONFIG;
    }
    return hipGetLastError() == hipSuccess ? MG_OK : MG_ERR_HIP;
}

}  // namespace mg
