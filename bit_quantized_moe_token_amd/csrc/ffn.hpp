// Shared declarations of the expert-FFN kernels (device helpers, argument
// block and host-side launchers).
#pragma once
#include <algorithm>
#include "common.hpp"

namespace moeq {

// Tokens per chunk of the weight-streaming kernels (up to two 16-row MFMA
// tiles).  A 64-token class (four tiles) needs twice the LDS and registers,
// which leaves one or two workgroups per CU; two 32-token chunks that each
// read the weights are faster at every size measured.
constexpr int kMT = 32;
constexpr int kSubPerChunk = kMT / 16;   // 16-token tiles per chunk
constexpr int kTiledM = 128;       // tokens per token tile of the tiled kernels
constexpr int kStripsPerWG = 4;    // one 16-row strip per wave

struct FfnArgs {
  const BlockDesc *desc;
  const int32_t *offsets;
  const int32_t *sorted_pairs;
  const uint16_t *x;
  const float *gates;
  const int32_t *pair_pos;
  int E, H, I, k, T, n_comp;
  int r, rs, Rp, Rsp, RZ;
  int comp_on;
  int G, fmt;
  float *zp_gu;     // [ks_gu][P][2][RZ] fp32 partial V x (summed by the consumer)
  float *zp_d;      // [ks_d][P][RZ] fp32 partial V_down h
  int ks_gu, ks_d;  // K splits of the two projections
  int64_t ks_stride_gu, ks_stride_d;   // floats between consecutive splits
  uint16_t *h;      // [P][I] fp16
  float *ypart;     // [splits][P][H] fp32
  int splits;
  int P;
  int nsub_max;     // largest number of 16-token tiles a chunk can have
};

struct Chunk {
  int e, m0, cnt, base;
};

// Chunk c of the expert-major chunk list (each expert's tokens cut into
// pieces of MT): expert, first token within the expert, token count and
// first sorted position.  Wave-uniform; false when c is past the end.
template <int MT = kMT>
__device__ __forceinline__ bool find_chunk(const int32_t *__restrict__ off, int E, int c, Chunk *out) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int b = 0; b < E; b += kWave) {
    const int e = b + lane;
    const int cnt = e < E ? off[e + 1] - off[e] : 0;
    const int nc = (cnt + MT - 1) / MT;
    int incl = nc;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += t;
    }
    const int excl = carry + incl - nc;
    const uint64_t hit = __ballot(c >= excl && c < excl + nc);
    if (hit) {
      // every lane holds the same values; readfirstlane makes that visible
      // to the compiler so they live in scalar registers
      const int src = __builtin_ctzll(hit);
      const int ex = __builtin_amdgcn_readfirstlane(__shfl(excl, src, kWave));
      const int cn = __builtin_amdgcn_readfirstlane(__shfl(cnt, src, kWave));
      out->e = __builtin_amdgcn_readfirstlane(b + src);
      out->m0 = (c - ex) * MT;
      out->cnt = std::min(MT, cn - out->m0);
      out->base = off[out->e] + out->m0;
      return true;
    }
    carry += __shfl(incl, kWave - 1, kWave);
  }
  return false;
}

__device__ __forceinline__ f16x8 load_a(const uint16_t *p) {
  return __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(p));
}

// Upper bound of the number of chunks of MT pairs for T tokens, top-k, E
// experts (an expert holds at most T pairs).
inline int max_chunks(int E, int T, int k, int MT = kMT) {
  const int64_t P = (int64_t)T * k;
  const int64_t a = (int64_t)E * ((T + MT - 1) / MT);
  const int64_t act = std::min<int64_t>(E, P);
  const int64_t b = (P + act * (MT - 1)) / MT;
  return (int)std::max<int64_t>(0, std::min(a, b));
}

// Launchers (stream.hip, lowrank.hip).
void launch_gateup_stream(const FfnArgs &a, int grid, hipStream_t s);
void launch_down_stream(const FfnArgs &a, int grid, hipStream_t s);
void launch_lowrank_project(const FfnArgs &a, int mode, dim3 grid, hipStream_t s);
void launch_combine(const FfnArgs &a, void *y, bool f32, hipStream_t s);
void launch_tiled_gateup(const FfnArgs &a, int grid, hipStream_t s);   // tiled_gu.hip
void launch_tiled_down(const FfnArgs &a, int grid, hipStream_t s);     // tiled_dn.hip

}  // namespace moeq
