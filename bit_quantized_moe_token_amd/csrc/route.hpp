// Device routines of the top-k routing and the token -> expert counting
// sort, shared by the routing kernels and the fused front kernel of the
// expert FFN (routing beside the low-rank projection in one launch).
#pragma once
#include "common.hpp"

namespace moeq {

constexpr int kMaxE = 256;
constexpr int kRouteTokens = 16;   // most tokens one routing workgroup takes

struct Cand {
  float v;
  int id;
};

__device__ __forceinline__ Cand better(Cand a, Cand b) {
  return (a.v > b.v || (a.v == b.v && a.id < b.id)) ? a : b;
}

// c against its partner lane under one DPP lane permutation (ctrl: a DPP
// control constant; every lane of a row is a valid source).
template <int CTRL>
__device__ __forceinline__ Cand dpp_better(Cand c) {
  Cand o;
  o.v = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, c.v), CTRL, 0xf, 0xf, true));
  o.id = __builtin_amdgcn_mov_dpp(c.id, CTRL, 0xf, 0xf, true);
  return better(c, o);
}

// Wave-wide best candidate, the same in every lane.  `better` is a total
// order on (value desc, id asc), so the result does not depend on the
// reduction tree: within each 16-lane row by DPP exchanges (quad swaps,
// then half-row and row mirrors: every lane ends with its row's best),
// then across the four rows through their first lanes.
__device__ __forceinline__ Cand wave_argmax(Cand c) {
  c = dpp_better<0xb1>(c);    // quad_perm [1,0,3,2]
  c = dpp_better<0x4e>(c);    // quad_perm [2,3,0,1]
  c = dpp_better<0x141>(c);   // row_half_mirror
  c = dpp_better<0x140>(c);   // row_mirror
  Cand r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    r[q].v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c.v), 16 * q));
    r[q].id = __builtin_amdgcn_readlane(c.id, 16 * q);
  }
  return better(better(r[0], r[1]), better(r[2], r[3]));
}

constexpr int kSlots = kMaxE / kWave;   // logits (and selected slots) per lane

// Logits of token t: lane l holds experts l + 64 s.
__device__ __forceinline__ void load_logits(const float *__restrict__ logits, int t, int E, float *v) {
  const int lane = threadIdx.x & 63;
  const float *row = logits + (int64_t)t * E;
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const int e = lane + s * kWave;
    v[s] = e < E ? row[e] : 0.0f;
  }
}

// Top-k of token t by one wave from its logits v: k rounds of a wave-wide
// argmax, gates in fp32.  The selected ids and logits stay in registers
// (slot j with lane j % 64) until all rounds are done, so no round waits
// for memory; then lanes j < k write slot j (and, if given, count it in
// the LDS histogram and copy its id to LDS).
__device__ __forceinline__ void topk_token(const float *v, int t, int E, int k, int32_t *__restrict__ ids,
                                           float *__restrict__ gates, int *s_hist, int *s_ids) {
  const int lane = threadIdx.x & 63;
  uint32_t taken = 0;
  float top0 = 0.0f, denom = 0.0f;
  float sel[kSlots];   // logit of slot j kept by lane j % 64
  int sid[kSlots];     // its expert id
#pragma unroll
  for (int s = 0; s < kSlots; ++s) { sel[s] = 0.0f; sid[s] = 0; }
  for (int j = 0; j < k; ++j) {
    Cand c{-__builtin_inff(), 0x7fffffff};
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      const int e = lane + s * kWave;
      if (e < E && !((taken >> s) & 1u)) c = better(c, Cand{v[s], e});
    }
    c = wave_argmax(c);                       // wave-uniform winner
    if ((c.id & 63) == lane) taken |= 1u << (c.id >> 6);
    if (j == 0) top0 = c.v;
    denom += __expf(c.v - top0);
    if ((j & 63) == lane) { sel[j >> 6] = c.v; sid[j >> 6] = c.id; }
  }
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const int j = lane + s * kWave;
    if (j < k) {
      ids[(int64_t)t * k + j] = sid[s];
      gates[(int64_t)t * k + j] = __expf(sel[s] - top0) / denom;
      if (s_hist) atomicAdd(&s_hist[sid[s]], 1);
      if (s_ids) s_ids[t * k + j] = sid[s];
    }
  }
}

// Tokens t0 + i * step < t1 (i < NT) by one wave: every token's logits
// are requested first, so the wave waits for memory once, not per token
// and not per round.
template <int NT>
__device__ __forceinline__ void topk_tokens(const float *__restrict__ logits, int t0, int t1, int step, int E, int k,
                                            int32_t *__restrict__ ids, float *__restrict__ gates, int *s_hist,
                                            int *s_ids = nullptr) {
  float v[NT][kSlots];
#pragma unroll
  for (int i = 0; i < NT; ++i)
    if (t0 + i * step < t1) load_logits(logits, t0 + i * step, E, v[i]);
  // all loads done here: the compiler then knows that no later wait is
  // needed (it would otherwise wait on each token's stores)
  vm_wait<0>();
#pragma unroll
  for (int i = 0; i < NT; ++i)
    if (t0 + i * step < t1) topk_token(v[i], t0 + i * step, E, k, ids, gates, s_hist, s_ids);
}

// LDS of one routing workgroup of NW waves.
template <int NW>
struct RouteLds {
  int count[kMaxE];
  int off[kMaxE + 1];
  int run[kMaxE];
  int wave[NW][kMaxE];
  int ids[kRouteTokens * kMaxE];   // the pairs' expert ids
};

// Outputs of routing (the moeq_routing arrays).
struct RouteOut {
  const float *logits;
  int32_t *ids;
  float *gates;
  int32_t *offsets;
  int32_t *sorted_pairs;
  int32_t *pair_pos;
};

// Routing of up to kRouteTokens tokens by one workgroup of NTH threads
// (every thread of the workgroup calls it).
// Phase 1: top-k + gates, kRouteTokens / NW tokens per wave; the histogram
//          and the ids also go to LDS, so the later phases read nothing
//          back from memory.
// Phase 2: exclusive scan of the histogram -> expert offsets.
// Phase 3: pairs in chunks of NTH in ascending pair id; a pair's rank among
//          equal experts inside its wave comes from ballots over the expert
//          id bits (peer mask); across waves and chunks from per-wave
//          counters in LDS.  Every slot is computed, none is found by
//          atomics, so the result is deterministic.
template <int NTH>
__device__ __forceinline__ void route_block(const RouteOut &o, int T, int E, int k, RouteLds<NTH / kWave> &s) {
  constexpr int NW = NTH / kWave;
  static_assert(kRouteTokens % NW == 0, "each wave takes the same number of tokens");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < kMaxE; e += NTH) { s.count[e] = 0; s.run[e] = 0; }
  __syncthreads();

  topk_tokens<kRouteTokens / NW>(o.logits, wave, T, NW, E, k, o.ids, o.gates, s.count, s.ids);
  __syncthreads();

  const int P = T * k;
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < E; base += kWave) {
      const int e = base + lane;
      const int c = e < E ? s.count[e] : 0;
      int incl = c;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int v = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += v;
      }
      if (e < E) s.off[e] = carry + incl - c;
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) s.off[E] = carry;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += NTH) o.offsets[e] = s.off[e];

  for (int base = 0; base < P; base += NTH) {
    const int p = base + tid;
    const bool valid = p < P;
    const int e = valid ? s.ids[p] : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t bal = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? bal : ~bal;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & below);
    const bool leader = valid && (peers & below) == 0;
    for (int x = tid; x < NW * kMaxE; x += NTH) (&s.wave[0][0])[x] = 0;
    __syncthreads();
    if (leader) s.wave[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int before = s.run[e];
      for (int w = 0; w < wave; ++w) before += s.wave[w][e];
      const int pos = s.off[e] + before + rank;
      o.sorted_pairs[pos] = p;
      o.pair_pos[p] = pos;
    }
    __syncthreads();
    for (int x = tid; x < E; x += NTH) {
      int add = 0;
      for (int w = 0; w < NW; ++w) add += s.wave[w][x];
      s.run[x] += add;
    }
    __syncthreads();
  }
}

}  // namespace moeq
