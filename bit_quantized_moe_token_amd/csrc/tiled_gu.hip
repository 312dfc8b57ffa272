// Instantiation of the tiled gate/up kernels (see tiled.hpp).
#include "tiled.hpp"

namespace moeq {

void launch_tiled_gateup(const FfnArgs &a, int grid, hipStream_t s) {
  if (a.fmt == MOEQ_FMT_BITPLANE)
    hipLaunchKernelGGL((tiled_gateup_kernel<1, true>), dim3(grid), dim3(64 * kTiledWaves), TStages<true>::kLaunchGU, s, a);
  else if (a.G == 64)
    hipLaunchKernelGGL((tiled_gateup_kernel<2, false>), dim3(grid), dim3(64 * kTiledWaves), TStages<false>::kLaunchGU, s, a);
  else
    hipLaunchKernelGGL((tiled_gateup_kernel<1, false>), dim3(grid), dim3(64 * kTiledWaves), TStages<false>::kLaunchGU, s, a);
}

}  // namespace moeq
