// Instantiation of the weight-streaming gateup kernels for one layer class
// (see stream.hpp).
#include "stream.hpp"

namespace moeq {

void launch_gateup_plane(const FfnArgs &a, int grid, hipStream_t s) {
  launch_gateup_class<1, true>(a, grid, s);
}

}  // namespace moeq
