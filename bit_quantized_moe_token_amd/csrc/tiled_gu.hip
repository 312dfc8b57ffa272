// Instantiation of the tiled gate/up kernels (see tiled.hpp).
#include "tiled.hpp"

namespace moeq {

void launch_tiled_gateup(const FfnArgs &a, int grid, hipStream_t s) {
  if (a.G == 64)
    hipLaunchKernelGGL((tiled_gateup_kernel<2>), dim3(grid), dim3(64 * kTiledWaves), kTiledLdsLaunch, s, a);
  else
    hipLaunchKernelGGL((tiled_gateup_kernel<1>), dim3(grid), dim3(64 * kTiledWaves), kTiledLdsLaunch, s, a);
}

}  // namespace moeq
