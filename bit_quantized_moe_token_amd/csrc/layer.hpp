// Packed-layer handle and tiled-layout index helpers (host + device).
#pragma once
#include <vector>
#include "common.hpp"

namespace moeq {

// Bytes per lane per tile of the code region: 4*b for INT, 4 per bit-plane.
__host__ __device__ inline int lane_tile_bytes(int fmt, int bits) {
  return fmt == MOEQ_FMT_INT ? 4 * bits : 4;
}

// Byte offset of lane l's data for tile t of strip s in a code region whose
// lanes hold W bytes per tile.  Tiles are grouped by four; inside a group a
// lane's bytes for the group's tiles are contiguous.  (Bit-plane regions,
// W = 4: one 16-byte chunk per lane per full group.)
__host__ __device__ inline uint64_t code_offset(int s, int t, int l, int n_kt, int W) {
  const int g4 = t >> 2, tl = t & 3;
  const int c = (n_kt - 4 * g4) < 4 ? (n_kt - 4 * g4) : 4;
  return (uint64_t)s * n_kt * 64 * W + (uint64_t)g4 * 256 * W + (uint64_t)l * c * W +
         (uint64_t)tl * W;
}

// Byte offset of dword e (0 <= e < B) of tile t, lane l, strip s of an INT
// code region (B dwords per lane per tile).  In a full group of four tiles
// the lane's 4*B dwords d = 4*tl... are split into B 16-byte chunks
// (dwords 4i..4i+3, d = tl*B + e) and chunk i of all 64 lanes is
// contiguous, so every 128-bit load instruction of a wave reads 1 KiB of
// consecutive bytes.  A ragged last group keeps the lane-contiguous layout.
__host__ __device__ inline uint64_t int_word_offset(int s, int t, int l, int e, int n_kt, int B) {
  const int g4 = t >> 2, tl = t & 3;
  const int c = (n_kt - 4 * g4) < 4 ? (n_kt - 4 * g4) : 4;
  const uint64_t base = (uint64_t)s * n_kt * 256 * B + (uint64_t)g4 * 1024 * B;
  if (c == 4) {
    const int d = tl * B + e;
    return base + (uint64_t)((d >> 2) * 64 + l) * 16 + (d & 3) * 4;
  }
  return base + (uint64_t)l * c * 4 * B + (uint64_t)tl * 4 * B + e * 4;
}

// Element index of the scale / zero of (strip s, tile t, row r, group gi in
// the tile); gpt = groups per tile (128 / G).
__host__ __device__ inline uint64_t meta_index(int s, int t, int r, int gi, int n_kt, int gpt) {
  const int g4 = t >> 2, tl = t & 3;
  const int c = (n_kt - 4 * g4) < 4 ? (n_kt - 4 * g4) : 4;
  return (uint64_t)s * n_kt * 16 * gpt + (uint64_t)g4 * 64 * gpt + (uint64_t)r * c * gpt +
         (uint64_t)tl * gpt + gi;
}

// Element index of LUT entry j of (strip s, tile t, row r); nq = 2^q.
__host__ __device__ inline uint64_t lut_index(int s, int t, int r, int j, int n_kt, int nq) {
  return ((uint64_t)s * n_kt + t) * 16 * nq + (uint64_t)r * nq + j;
}

}  // namespace moeq

struct moeq_layer {
  moeq::LayerDims dims;
  uint8_t *buf;
  size_t bytes;
  moeq::BlockDesc *d_desc;                 // device table (inside buf)
  std::vector<moeq::BlockDesc> h_desc;     // host copy of the table
  std::vector<uint8_t> bits;               // [E*3] committed q (b for INT)
  std::vector<size_t> block_alg_bytes;     // [E*3]
  std::vector<size_t> shared_alg_bytes;    // [groups*3]
  // bit-plane page table: planes [0, resident) of a block are in device
  // memory; desired is the bitwidth the runtime is moving the block to.
  // commit_ev is recorded after each commit of the block, copy_ev after
  // each release or reload; reload_pending marks a reload no commit has
  // waited for yet.  (Host-side state, enqueue order; events exist for
  // bit-plane layers only.)
  std::vector<uint8_t> resident, desired, reload_pending;   // [E*3]
  std::vector<hipEvent_t> commit_ev, copy_ev;                // [E*3]
  ~moeq_layer() {
    for (hipEvent_t e : commit_ev) (void)hipEventDestroy(e);
    for (hipEvent_t e : copy_ev) (void)hipEventDestroy(e);
  }
};
