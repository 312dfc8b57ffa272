// Top-k routing and the token -> expert counting sort, in one workgroup.
//
// Top-k with softmax gates over the selected logits (router-guided top-n
// compensation, "Bandwidth-Efficient Adaptive Mixture-of-Experts via
// Low-Rank Compensation", abstract, presupposes a per-token top-k list) and a
// stable counting sort of the (token, slot) pairs by expert with prefix-sum
// offsets (MxMoE abstract: uneven expert activation makes per-expert work
// heterogeneous, so experts get contiguous, variable-length row ranges).
//
// Phase 1: one wave per token; k rounds of a wave-wide argmax over
//          (logit desc, expert id asc).
// Phase 2: LDS histogram -> exclusive scan -> expert_offsets.
// Phase 3: pairs in chunks of 1024 in ascending pair id; a pair's rank among
//          equal experts inside its wave comes from ballots over the expert
//          id bits (peer mask) and mbcnt; across waves and chunks from
//          per-wave counters in LDS.  Every pair's slot is computed, none is
//          found by atomics, so the result is deterministic.
#include "common.hpp"

namespace moeq {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kMaxE = 256;

struct Cand {
  float v;
  int id;
};

__device__ __forceinline__ Cand better(Cand a, Cand b) {
  return (a.v > b.v || (a.v == b.v && a.id < b.id)) ? a : b;
}

__device__ __forceinline__ Cand wave_argmax(Cand c) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Cand o;
    o.v = __shfl_xor(c.v, off, kWave);
    o.id = __shfl_xor(c.id, off, kWave);
    c = better(c, o);
  }
  return c;
}

__global__ void __launch_bounds__(kRouteThreads)
route_kernel(const float *__restrict__ logits, int T, int E, int k, int32_t *__restrict__ ids,
             float *__restrict__ gates, int32_t *__restrict__ offsets,
             int32_t *__restrict__ sorted_pairs, int32_t *__restrict__ pair_pos) {
  __shared__ int s_count[kMaxE];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_run[kMaxE];
  __shared__ int s_wave[kRouteWaves][kMaxE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < kMaxE; e += kRouteThreads) { s_count[e] = 0; s_run[e] = 0; }

  // ---- phase 1: top-k + gates, one wave per token
  for (int t = wave; t < T; t += kRouteWaves) {
    const float *row = logits + (int64_t)t * E;
    float v[kMaxE / kWave];
    uint32_t taken = 0;
#pragma unroll
    for (int s = 0; s < kMaxE / kWave; ++s) {
      const int e = lane + s * kWave;
      v[s] = e < E ? row[e] : 0.0f;
    }
    float top0 = 0.0f, denom = 0.0f;
    float sel[kMaxE / kWave];   // logit of slot j kept by lane j % 64
#pragma unroll
    for (int s = 0; s < kMaxE / kWave; ++s) sel[s] = 0.0f;
    for (int j = 0; j < k; ++j) {
      Cand c{-__builtin_inff(), 0x7fffffff};
#pragma unroll
      for (int s = 0; s < kMaxE / kWave; ++s) {
        const int e = lane + s * kWave;
        if (e < E && !((taken >> s) & 1u)) c = better(c, Cand{v[s], e});
      }
      c = wave_argmax(c);                       // wave-uniform winner
      if ((c.id & 63) == lane) taken |= 1u << (c.id >> 6);
      if (j == 0) top0 = c.v;
      denom += __expf(c.v - top0);
      if ((j & 63) == lane) sel[j >> 6] = c.v;
      if (lane == 0) ids[(int64_t)t * k + j] = c.id;
    }
#pragma unroll
    for (int s = 0; s < kMaxE / kWave; ++s) {
      const int j = lane + s * kWave;
      if (j < k) gates[(int64_t)t * k + j] = __expf(sel[s] - top0) / denom;
    }
  }
  __syncthreads();

  // ---- phase 2: histogram + exclusive scan
  const int P = T * k;
  for (int p = tid; p < P; p += kRouteThreads) atomicAdd(&s_count[ids[p]], 1);
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < E; base += kWave) {
      const int e = base + lane;
      const int c = e < E ? s_count[e] : 0;
      int incl = c;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += o;
      }
      if (e < E) s_off[e] = carry + incl - c;
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) s_off[E] = carry;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += kRouteThreads) offsets[e] = s_off[e];

  // ---- phase 3: stable placement
  for (int base = 0; base < P; base += kRouteThreads) {
    const int p = base + tid;
    const bool valid = p < P;
    const int e = valid ? ids[p] : 0;
    // lanes of this wave holding the same expert
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t bal = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? bal : ~bal;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & below);
    const bool leader = valid && (peers & below) == 0;
    for (int x = tid; x < kRouteWaves * kMaxE; x += kRouteThreads) (&s_wave[0][0])[x] = 0;
    __syncthreads();
    if (leader) s_wave[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int before = s_run[e];
      for (int w = 0; w < wave; ++w) before += s_wave[w][e];
      const int pos = s_off[e] + before + rank;
      sorted_pairs[pos] = p;
      pair_pos[p] = pos;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kRouteThreads) {
      int add = 0;
      for (int w = 0; w < kRouteWaves; ++w) add += s_wave[w][x];
      s_run[x] += add;
    }
    __syncthreads();
  }
}

}  // namespace moeq

using namespace moeq;

MOEQ_API moeq_status moeq_route_workspace_size(int32_t T, int32_t E, int32_t k, size_t *bytes) {
  if (!bytes) return fail(MOEQ_ERR_INVALID, "route_workspace_size: null output");
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E)
    return fail(MOEQ_ERR_INVALID, "route_workspace_size: T=%d E=%d k=%d invalid", T, E, k);
  *bytes = 0;
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_route(const float *logits, int32_t T, int32_t E, int32_t k,
                                const moeq_routing *out, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (!out) return fail(MOEQ_ERR_INVALID, "route: null routing output");
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E)
    return fail(MOEQ_ERR_INVALID, "route: T=%d E=%d k=%d invalid (need 1 <= k <= E <= 256)", T, E, k);
  if ((int64_t)T * k > (int64_t)0x7fffffff) return fail(MOEQ_ERR_UNSUPPORTED, "route: T*k too large");
  if (!out->expert_offsets || (T > 0 && (!logits || !out->topk_ids || !out->topk_gates ||
                                         !out->sorted_pairs || !out->pair_pos)))
    return fail(MOEQ_ERR_INVALID, "route: null pointer");
  prof_begin("route", stream);
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), 0, stream, logits, T, E, k,
                     out->topk_ids, out->topk_gates, out->expert_offsets, out->sorted_pairs,
                     out->pair_pos);
  prof_end("route", stream);
  return check_launch("route");
}
