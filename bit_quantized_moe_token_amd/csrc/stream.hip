// Dispatch of the weight-streaming kernels by layer class (INT group 128,
// INT group 64, bit-plane).
#include "stream.hpp"

namespace moeq {

void launch_gateup_stream(const FfnArgs &a, int grid, hipStream_t s) {
  if (a.fmt == MOEQ_FMT_BITPLANE) launch_gateup_plane(a, grid, s);
  else if (a.G == 64) launch_gateup_g64(a, grid, s);
  else launch_gateup_g128(a, grid, s);
}

void launch_down_stream(const FfnArgs &a, int grid, hipStream_t s) {
  if (a.fmt == MOEQ_FMT_BITPLANE) launch_down_plane(a, grid, s);
  else if (a.G == 64) launch_down_g64(a, grid, s);
  else launch_down_g128(a, grid, s);
}

}  // namespace moeq
