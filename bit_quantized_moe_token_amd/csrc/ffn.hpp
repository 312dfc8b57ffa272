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
  float *zp_gu;     // [ks_gu][P][2][RZ] fp32 partial V x (summed by the consumer), by sorted
                    // position; with z_tok [ks_gu][T][E][2][RZ] by (token, expert), every pair
  int z_tok;
  float *zp_d;      // [ks_d][P][RZ] fp32 partial V_down h
  int ks_gu, ks_d;  // K splits of the two projections
  int64_t ks_stride_gu, ks_stride_d;   // floats between consecutive splits
  uint16_t *h;      // [P][I] fp16: h * 2^(kNormTop - eb), eb per (pair, 64-row block of I)
  int8_t *hblk;     // [P][hblk_stride] eb (h_block_exp), I/64 used per row
  int hblk_stride;  // bytes per row of hblk (I/64 rounded up to 16)
  uint16_t *hn;     // [P][I] fp16: h * 2^(kNormTop - eh), eh = the pair's largest eb
  int32_t *hexp;    // [P] eh (set to kHZero by the first launch, raised by the gate/up kernels)
  int32_t *xexp;    // [T] K of each token (x_norm_exp)
  uint16_t *xn;     // [T][H] x * 2^K, the activations the gate/up kernels read
  float *ypart;     // [splits][P][H] fp32, in units of 2^(eh - kNormTop) (the combine undoes it)
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

// ---- activation normalisation (see kNormTop).

// Exponent of a block of h with largest magnitude mx, as stored (int8):
// floor(log2 mx) clamped to [-127, 127], kHZero (-128) for an all-zero
// block.  h 2^(kNormTop - eb) then has its largest magnitude in
// [2^kNormTop, 2^(kNormTop+1)) (smaller where the clamp applies).
constexpr int kHZero = -128;
__device__ __forceinline__ int h_block_exp(float mx) {
  const int e = ilogb_f32(mx);
  return e == kNoExp ? kHZero : std::max(-127, std::min(127, e));
}

// x exponents of tokens t = wid, wid + nw, ...: one wave per token takes
// the largest |x| of the row (fp16 magnitude bits compare as integers),
// writes K = x_norm_exp of its exponent and the row x 2^K to xn.  The same
// waves set every pair's h exponent eh to kHZero, the start of the maximum
// that the gate/up kernels take over their blocks (h_pair_exp).
__device__ __forceinline__ void xexp_rows(const FfnArgs &a, int wid, int nw) {
  const int lane = threadIdx.x & 63;
  for (int i = wid * kWave + lane; i < a.P; i += nw * kWave) a.hexp[i] = kHZero;
  for (int t = wid; t < a.T; t += nw) {
    const uint16_t *row = a.x + (int64_t)t * a.H;
    uint32_t m = 0;
    for (int c = 8 * lane; c < a.H; c += 8 * kWave) {
      const u32x4 v = gld<u32x4>(row + c);
#pragma unroll
      for (int w = 0; w < 4; ++w) m = std::max(m, std::max(v[w] & 0x7fffu, (v[w] >> 16) & 0x7fffu));
    }
#pragma unroll
    for (int o = 32; o; o >>= 1) m = std::max(m, (uint32_t)__shfl_xor((int)m, o, kWave));
    const int K = x_norm_exp(ilogb_f16bits(m));
    if (lane == 0) a.xexp[t] = K;
    const uint32_t mul = f16x2_pow2(K);
    uint16_t *out = a.xn + (int64_t)t * a.H;
    for (int c = 8 * lane; c < a.H; c += 8 * kWave)
      *reinterpret_cast<u32x4 *>(out + c) = scale_f16x8(gld<u32x4>(row + c), mul);
  }
}

// eh of the pair at sorted position pos = the largest eb over its blocks:
// each gate/up workgroup raises it to the eb of the block it wrote (an
// integer maximum, so the result does not depend on the order).
__device__ __forceinline__ void h_pair_exp(const FfnArgs &a, int pos, int eb) { atomicMax(a.hexp + pos, eb); }

// x exponent of chunk row m (rows past the count repeat the last one).
__device__ __forceinline__ int row_kx(const FfnArgs &a, const Chunk &ch, int m) {
  return a.xexp[a.sorted_pairs[ch.base + std::min(m, ch.cnt - 1)] / a.k];
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

struct RouteOut;   // route.hpp

// Launchers (stream.hip, lowrank.hip).
void launch_gateup_stream(const FfnArgs &a, int grid, hipStream_t s);
void launch_down_stream(const FfnArgs &a, int grid, hipStream_t s);
void launch_lowrank_project(const FfnArgs &a, int mode, int jobs, hipStream_t s);   // jobs: 16-column jobs
void launch_front_routed(const FfnArgs &a, const RouteOut &ro, hipStream_t s);   // needs a.z_tok, a.T <= kRouteTokens
void launch_combine(const FfnArgs &a, void *y, bool f32, hipStream_t s);
void launch_xexp(const FfnArgs &a, hipStream_t s);    // x exponents alone (no gate/up projection)
void launch_hnorm(const FfnArgs &a, hipStream_t s);   // h renormalisation alone (no down projection)
void launch_tiled_gateup(const FfnArgs &a, int grid, hipStream_t s);   // tiled_gu.hip
void launch_tiled_down(const FfnArgs &a, int grid, hipStream_t s);     // tiled_dn.hip

}  // namespace moeq
