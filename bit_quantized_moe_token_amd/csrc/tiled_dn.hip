// Instantiation of the tiled down kernels (see tiled.hpp).
#include "tiled.hpp"

namespace moeq {

void launch_tiled_down(const FfnArgs &a, int grid, hipStream_t s) {
  if (a.G == 64)
    hipLaunchKernelGGL((tiled_down_kernel<2>), dim3(grid), dim3(64 * kTiledWaves), kTiledLdsBytes, s, a);
  else
    hipLaunchKernelGGL((tiled_down_kernel<1>), dim3(grid), dim3(64 * kTiledWaves), kTiledLdsBytes, s, a);
}

}  // namespace moeq
