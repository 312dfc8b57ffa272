// Instantiation of the tiled down kernels (see tiled.hpp).
#include "tiled.hpp"

namespace moeq {

void launch_tiled_down(const FfnArgs &a, int grid, hipStream_t s) {
  if (a.fmt == MOEQ_FMT_BITPLANE)
    hipLaunchKernelGGL((tiled_down_kernel<1, true>), dim3(grid), dim3(64 * kTiledWaves), TStages<true>::kLds, s, a);
  else if (a.G == 64)
    hipLaunchKernelGGL((tiled_down_kernel<2, false>), dim3(grid), dim3(64 * kTiledWaves), TStages<false>::kLds, s, a);
  else
    hipLaunchKernelGGL((tiled_down_kernel<1, false>), dim3(grid), dim3(64 * kTiledWaves), TStages<false>::kLds, s, a);
}

}  // namespace moeq
