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
  const int32_t *ids;   // [T][k] expert of each slot (read with shared factors only)
  int share;            // experts per shared-factor group (1 without shared factors)
  int E, H, I, k, T, n_comp;
  int r, rs, Rp, Rsp, RZ;
  int comp_on;
  int G, fmt;
  float *zp_gu;     // [ks_gu][P][2][RZ] fp32 partial V x (summed by the consumer), by sorted
                    // position; with z_tok [ks_gu][T][E][2][RZ] by (token, expert), every pair
  int z_tok;
  float *zp_d;      // [ks_d][P][RZ] fp32 partial V_down h (per-expert columns)
  float *zsh;       // [ks_d][P][k][Rsp] fp32: shared columns, row of the down leader of
                    // (token, group), sub-row = the member's slot (see slot_group)
  int32_t *dlead;   // [P] member mask of a down leader, 0 for the other pairs
  int64_t ks_stride_sh;
  int ks_gu, ks_d;  // K splits of the two projections
  int wt;            // the down projection runs in wave tiles (see lowrank_project_kernel)
  int64_t ks_stride_gu, ks_stride_d;   // floats between consecutive splits
  uint16_t *h;      // [P][I] fp16: h * 2^(kNormTop - eb), eb per (pair, 64-row block of I)
  int8_t *hblk;     // [P][hblk_stride] eb (h_block_exp), I/64 used per row
  int hblk_stride;  // bytes per row of hblk (I/64 rounded up to 16)
  uint16_t *hn;     // [P][I] fp16: h * 2^(kNormTop - eh), eh = the pair's largest eb
  int32_t *hexp;    // [P] eh by sorted position (set to kHZero by the first launch, raised by
                    // the gate/up kernels)
  int32_t *hexpf;   // [P] the same by pair id t*k + j
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
  for (int i = wid * kWave + lane; i < a.P; i += nw * kWave) a.hexp[i] = a.hexpf[i] = kHZero;
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

// eh of the pair p at sorted position pos = the largest eb over its
// blocks: each gate/up workgroup raises it to the eb of the block it wrote
// (an integer maximum, so the result does not depend on the order); kept
// by position and by pair id.
__device__ __forceinline__ void h_pair_exp(const FfnArgs &a, int pos, int p, int eb) {
  atomicMax(a.hexp + pos, eb);
  atomicMax(a.hexpf + p, eb);
}

// Shared factors (TileQ abstract: factors shared by a group of experts).
// The compensated slots of token t whose experts lie in group G, as a slot
// mask (n_comp <= 32 with shared factors), and the slot that carries the
// group's work for the token (its leader):
//   gate/up: the first member; it computes V_G x once for (t, G) and
//   writes it into the z rows of every member;
//   down (DOWN): the member m of largest g_m 2^eh_m (its key
//   eh_m + log2 g_m; ties to the lower slot).  U_G is applied once, in the
//   leader's row, to w' = sum over members m of f_m V_G hn_m with
//   f_m = g_m 2^eh_m / (g_lead 2^eh_lead) <= 1 (hn_m = h_m 2^(kNormTop -
//   eh_m)); the combine's factor g_lead 2^(eh_lead - kNormTop) for the
//   leader's row then gives sum_m g_m U_G V_G h_m, and w' never exceeds
//   the size of the z rows.
struct SlotGroup {
  uint32_t mask;
  int lead;       // slot
  int lead_pos;   // DOWN: sorted position of the leader
  float key;      // DOWN: the leader's key
};

__device__ __forceinline__ float down_key(float g, int eh) {
  return g > 0.f ? (float)eh + __builtin_log2f(g) : -__builtin_inff();
}

// Eight slots j0 .. j0 + 7 of a token (row = t * k) as loaded, every load
// issued before the first use (all indexed by pair id, so none waits for
// another): the experts, and for DOWN the positions, gates and h exponents.
struct SlotBatch {
  int id[8], pp[8], eh[8];
  float g[8];
};

// (the loads are unconditional, at slots clamped to n_comp - 1 >= 0, so
// that no branch separates them and nothing uses them before the fold;
// the fold skips the slots past n_comp)
template <bool DOWN>
__device__ __forceinline__ void slot_batch_load(const FfnArgs &a, int64_t row, int j0, SlotBatch &b) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t q = row + std::min(j0 + u, a.n_comp - 1);
    b.id[u] = a.ids[q];
    if (DOWN) {
      b.pp[u] = a.pair_pos[q];
      b.g[u] = a.gates[q];
      b.eh[u] = a.hexpf[q];
    } else {
      b.pp[u] = 0;
      b.g[u] = 0.f;
      b.eh[u] = 0;
    }
  }
}

template <bool DOWN>
__device__ __forceinline__ void slot_batch_fold(const FfnArgs &a, int j0, int G, SlotBatch b, SlotGroup &g) {
  // (the values pass through an empty asm here, so that the compiler does
  // not move their uses, and the wait for the loads, up to where they were
  // requested)
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    asm volatile("" : "+v"(b.id[u]), "+v"(b.pp[u]), "+v"(b.g[u]), "+v"(b.eh[u]));
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (j0 + u >= a.n_comp || b.id[u] / a.share != G) continue;
    g.mask |= 1u << (j0 + u);
    if (!DOWN) {
      if (g.lead < 0) g.lead = j0 + u;
    } else {
      const float key = down_key(b.g[u], b.eh[u]);
      if (g.lead < 0 || key > g.key) {
        g.key = key;
        g.lead = j0 + u;
        g.lead_pos = b.pp[u];
      }
    }
  }
}

// The group of (t, G), from slots 0..7 loaded earlier (first) and the
// rest loaded here.
template <bool DOWN>
__device__ __forceinline__ SlotGroup slot_group_from(const FfnArgs &a, int t, int G, const SlotBatch &first) {
  SlotGroup g{0u, -1, 0, -__builtin_inff()};
  slot_batch_fold<DOWN>(a, 0, G, first, g);
  const int64_t row = (int64_t)t * a.k;
  for (int j0 = 8; j0 < a.n_comp; j0 += 8) {
    SlotBatch b;
    slot_batch_load<DOWN>(a, row, j0, b);
    slot_batch_fold<DOWN>(a, j0, G, b, g);
  }
  return g;
}

// f_m of a member with key `key` in a group whose leader has key `lead`
// (0 when every member's gate is 0).
__device__ __forceinline__ float down_factor(float key, float lead) {
  return lead == -__builtin_inff() ? 0.f : __builtin_exp2f(key - lead);
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
