// Top-k routing and the token -> expert counting sort: in one workgroup for
// up to 64 tokens, else in 64-token segments (per-segment counts, then
// offsets and placement per segment).
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

// Top-k of token t by one wave: k rounds of a wave-wide argmax, gates in
// fp32; lane 0 writes ids (and counts them in an LDS histogram if given).
__device__ __forceinline__ void topk_token(const float *__restrict__ logits, int t, int E, int k,
                                           int32_t *__restrict__ ids, float *__restrict__ gates,
                                           int *s_hist) {
  const int lane = threadIdx.x & 63;
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
    if (lane == 0) {
      ids[(int64_t)t * k + j] = c.id;
      if (s_hist) atomicAdd(&s_hist[c.id], 1);
    }
  }
#pragma unroll
  for (int s = 0; s < kMaxE / kWave; ++s) {
    const int j = lane + s * kWave;
    if (j < k) gates[(int64_t)t * k + j] = __expf(sel[s] - top0) / denom;
  }
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
  for (int t = wave; t < T; t += kRouteWaves) topk_token(logits, t, E, k, ids, gates, nullptr);
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


// ---- many tokens: segments of kSegTokens tokens, two kernels.
constexpr int kSegThreads = 256;
constexpr int kSegWaves = kSegThreads / kWave;
constexpr int kSegTokens = 64;

// Segment blockIdx.x: top-k of its tokens (16 waves, one per token) and
// its per-expert pair counts seg_count[seg][e].
__global__ void __launch_bounds__(kRouteThreads)
route_topk_kernel(const float *__restrict__ logits, int T, int E, int k, int32_t *__restrict__ ids,
                  float *__restrict__ gates, int32_t *__restrict__ seg_count) {
  __shared__ int s_hist[kMaxE];
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int e = tid; e < kMaxE; e += kRouteThreads) s_hist[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kSegTokens, t1 = std::min(T, t0 + kSegTokens);
  for (int t = t0 + wave; t < t1; t += kRouteWaves) topk_token(logits, t, E, k, ids, gates, s_hist);
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) seg_count[(int64_t)blockIdx.x * E + e] = s_hist[e];
}

// Segment blockIdx.x: expert offsets from every segment's counts (segment 0
// writes them), this segment's first slot per expert (pairs of earlier
// segments come first), then the stable placement of its pairs in
// ascending pair id (ballot peer masks inside a wave, per-wave counts
// across waves and chunks).
__global__ void __launch_bounds__(kSegThreads)
route_place_kernel(const int32_t *__restrict__ ids, int T, int E, int k, const int32_t *__restrict__ seg_count,
                   int nseg, int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_pairs,
                   int32_t *__restrict__ pair_pos) {
  __shared__ int s_tot[kMaxE];
  __shared__ int s_base[kMaxE];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_run[kMaxE];
  __shared__ int s_wave[kSegWaves][kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = blockIdx.x;
  for (int e = tid; e < E; e += kSegThreads) {
    int tot = 0, before = 0;
#pragma unroll 8
    for (int g = 0; g < nseg; ++g) {
      const int c = seg_count[(int64_t)g * E + e];
      tot += c;
      before += g < seg ? c : 0;
    }
    s_tot[e] = tot;
    s_base[e] = before;
    s_run[e] = 0;
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < E; base += kWave) {
      const int e = base + lane;
      const int c = e < E ? s_tot[e] : 0;
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
  if (seg == 0)
    for (int e = tid; e <= E; e += kSegThreads) offsets[e] = s_off[e];
  for (int e = tid; e < E; e += kSegThreads) s_base[e] += s_off[e];
  __syncthreads();
  const int p0 = seg * kSegTokens * k, p1 = std::min(T, (seg + 1) * kSegTokens) * k;
  for (int base = p0; base < p1; base += kSegThreads) {
    const int p = base + tid;
    const bool valid = p < p1;
    const int e = valid ? ids[p] : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t bal = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? bal : ~bal;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & below);
    const bool leader = valid && (peers & below) == 0;
    for (int x = tid; x < kSegWaves * kMaxE; x += kSegThreads) (&s_wave[0][0])[x] = 0;
    __syncthreads();
    if (leader) s_wave[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int before = s_run[e];
      for (int w = 0; w < wave; ++w) before += s_wave[w][e];
      const int pos = s_base[e] + before + rank;
      sorted_pairs[pos] = p;
      pair_pos[p] = pos;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kSegThreads) {
      int add = 0;
      for (int w = 0; w < kSegWaves; ++w) add += s_wave[w][x];
      s_run[x] += add;
    }
    __syncthreads();
  }
}

static inline int route_segments(int T) { return (T + kSegTokens - 1) / kSegTokens; }

// Routing mass (PagedWeight review summary: routing-mass buckets protect
// frequently used experts): m_e = sum of the gates of expert e's pairs.
// One wave per expert: lane-strided partial sums over the expert's sorted
// pairs, then a fixed xor-shuffle tree, so the result is deterministic.
// bucket_e = number of edges <= m_e.
constexpr int kMaxEdges = 8;
struct MassEdges {
  float v[kMaxEdges];
  int n;
};

__global__ void __launch_bounds__(256)
route_mass_kernel(const float *__restrict__ gates, const int32_t *__restrict__ offsets,
                  const int32_t *__restrict__ sorted_pairs, int E, MassEdges ed, float *__restrict__ mass,
                  int32_t *__restrict__ bucket) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const int lo = offsets[e], hi = offsets[e + 1];
  float acc = 0.f;
  for (int pos = lo + lane; pos < hi; pos += kWave) acc += gates[sorted_pairs[pos]];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, kWave);
  if (lane == 0) {
    mass[e] = acc;
    if (bucket) {
      int b = 0;
      for (int i = 0; i < ed.n; ++i) b += ed.v[i] <= acc ? 1 : 0;
      bucket[e] = b;
    }
  }
}

}  // namespace moeq

using namespace moeq;

// Up to kRouteSingleMax tokens: the single-workgroup kernel (one launch;
// its waves take the tokens in turn); more: segments, with per-segment
// counts in the workspace.
constexpr int kRouteSingleMax = 64;
static inline bool route_single(int T) { return T <= kRouteSingleMax; }
static inline size_t route_ws_bytes(int T, int E) {
  return route_single(T) ? 0 : (size_t)route_segments(T) * E * sizeof(int32_t);
}

MOEQ_API moeq_status moeq_route_workspace_size(int32_t T, int32_t E, int32_t k, size_t *bytes) {
  if (!bytes) return fail(MOEQ_ERR_INVALID, "route_workspace_size: null output");
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E)
    return fail(MOEQ_ERR_INVALID, "route_workspace_size: T=%d E=%d k=%d invalid", T, E, k);
  *bytes = route_ws_bytes(T, E);
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_route(const float *logits, int32_t T, int32_t E, int32_t k,
                                const moeq_routing *out, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
  if (!out) return fail(MOEQ_ERR_INVALID, "route: null routing output");
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E)
    return fail(MOEQ_ERR_INVALID, "route: T=%d E=%d k=%d invalid (need 1 <= k <= E <= 256)", T, E, k);
  if ((int64_t)T * k > (int64_t)0x7fffffff) return fail(MOEQ_ERR_UNSUPPORTED, "route: T*k too large");
  if (!out->expert_offsets || (T > 0 && (!logits || !out->topk_ids || !out->topk_gates ||
                                         !out->sorted_pairs || !out->pair_pos)))
    return fail(MOEQ_ERR_INVALID, "route: null pointer");
  const size_t need = route_ws_bytes(T, E);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(MOEQ_ERR_WORKSPACE, "route: workspace has %zu bytes, needs %zu", ws_bytes, need);
  prof_begin("route", stream);
  const int nseg = route_segments(T);
  if (route_single(T)) {
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), 0, stream, logits, T, E, k,
                       out->topk_ids, out->topk_gates, out->expert_offsets, out->sorted_pairs,
                       out->pair_pos);
  } else {
    int32_t *cnt = static_cast<int32_t *>(ws);
    hipLaunchKernelGGL(route_topk_kernel, dim3(nseg), dim3(kRouteThreads), 0, stream, logits, T, E, k,
                       out->topk_ids, out->topk_gates, cnt);
    hipLaunchKernelGGL(route_place_kernel, dim3(nseg), dim3(kSegThreads), 0, stream, out->topk_ids, T, E, k,
                       cnt, nseg, out->expert_offsets, out->sorted_pairs, out->pair_pos);
  }
  prof_end("route", stream);
  return check_launch("route");
}

MOEQ_API moeq_status moeq_route_mass(const moeq_routing *r, int32_t T, int32_t E, int32_t k, const float *edges,
                                     int32_t n_edges, float *mass, int32_t *bucket, hipStream_t stream) {
  if (!r) return fail(MOEQ_ERR_INVALID, "route_mass: null routing");
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E)
    return fail(MOEQ_ERR_INVALID, "route_mass: T=%d E=%d k=%d invalid", T, E, k);
  if (n_edges < 0 || n_edges > kMaxEdges || (n_edges > 0 && !edges))
    return fail(MOEQ_ERR_INVALID, "route_mass: n_edges=%d not in 0..%d (or null edges)", n_edges, kMaxEdges);
  MassEdges ed{};
  ed.n = n_edges;
  for (int i = 0; i < n_edges; ++i) {
    if (!(edges[i] == edges[i]) || (i > 0 && edges[i] < edges[i - 1]))
      return fail(MOEQ_ERR_INVALID, "route_mass: edges must be ascending and not NaN");
    ed.v[i] = edges[i];
  }
  if (!mass || !r->expert_offsets || (T > 0 && (!r->topk_gates || !r->sorted_pairs)))
    return fail(MOEQ_ERR_INVALID, "route_mass: null pointer");
  prof_begin("route_mass", stream);
  hipLaunchKernelGGL(route_mass_kernel, dim3((E + 3) / 4), dim3(256), 0, stream, r->topk_gates, r->expert_offsets,
                     r->sorted_pairs, E, ed, mass, bucket);
  prof_end("route_mass", stream);
  return check_launch("route_mass");
}
