// fp32 GEMM kernel (mg_f32.h) and its launcher.
#include "mg_table.h"
#include "mg_f32.h"

namespace mg {

using CfgF32 = F32Cfg<kF32TileM, kF32TileN, 2, 2, kF32SliceK, 4>;

mg_status launch_f32(bool epi, const KArgs& a, int64_t grid, hipStream_t s) {
    (void)hipGetLastError();
    if (epi)
        hipLaunchKernelGGL((gemm_f32_kernel<CfgF32, true>), dim3((unsigned)grid), dim3(CfgF32::NT), 0, s, a);
    else
        hipLaunchKernelGGL((gemm_f32_kernel<CfgF32, false>), dim3((unsigned)grid), dim3(CfgF32::NT), 0, s, a);
    return hipGetLastError() == hipSuccess ? MG_OK : MG_ERR_HIP;
}

}  // namespace mg
