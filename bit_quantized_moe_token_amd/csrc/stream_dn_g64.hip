// Instantiation of the weight-streaming down kernels for one layer class
// (see stream.hpp).
#include "stream.hpp"

namespace moeq {

void launch_down_g64(const FfnArgs &a, int grid, hipStream_t s) {
  launch_down_class<2, false>(a, grid, s);
}

}  // namespace moeq
