// Instantiation of the weight-streaming gateup kernels for one layer class
// (see stream.hpp).
#include "stream.hpp"

namespace moeq {

void launch_gateup_g64(const FfnArgs &a, int grid, hipStream_t s) {
  launch_gateup_class<2, false>(a, grid, s);
}

}  // namespace moeq
