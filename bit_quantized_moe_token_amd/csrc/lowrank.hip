// Skinny low-rank projections and the combine.
//
// z = V v for each compensated pair (MiLo abstract: low-rank compensators;
// TileQ abstract: factors shared by a group of experts, so a pair also
// gets the group's V_G v, once per (token, group) on the gate/up side;
// Bandwidth-Efficient Adaptive MoE abstract: only a token's top-n slots are
// compensated, the other rows of z are zero), and y_t = sum_j g_{t,j}
// y_pair(t, j) summed in slot order.
#include "common.hpp"
#include "ffn.hpp"
#include "route.hpp"

namespace moeq {

// Partial z[pos][slot] = V v over one K range for compensated pairs (zero
// for the others); the consumer kernels sum the ks partials in fixed order.
// One 16-token tile and NJ 16-column jobs per workgroup (NJ = 2, 4 or 8
// when many tokens leave no K split: each activation fragment then feeds
// every job, so the activations are read NJ times less often); 4 waves
// split the range and reduce through LDS in fixed order.
// grid.x = max_chunks * kSubPerChunk tiles, grid.y = (#blocks) * (Rp + Rsp) / 16 / NJ
// (+ 1 in modes 0 and 2), grid.z = ks.  mode 0: v = x[token] (gate/up
// blocks) of each routed pair; mode 2: the same for every (token, expert)
// pair (grid.x = ceil(T / 16) * E), which needs no routing; in both the
// extra y slice (blockIdx.y == njy) computes the tokens' x exponents
// instead.  mode 1: v = h of the pair, renormalised on the fly from its
// per-block exponents to the pair's exponent eh (final once the gate/up
// kernel has run); the workgroups of y slice 0 also store that
// renormalised h (hn), which the down kernels read.
// ROUTE (mode 2 only): one more y slice, whose first workgroup routes the
// tokens (route_block) while the others project; the projection of every
// (token, expert) pair needs no routing, so both fit in one launch.
// A tile none of whose pairs is compensated (router-guided top-n) loads
// no V and writes zero rows.
// SH: the layer has shared factors (the group bookkeeping is compiled in
// only then: its registers would cost the other layers occupancy).
// WT (mode 1, many pairs, no shared factors): each wave owns one 16-pair
// tile of a 64-pair chunk and the workgroup's whole K range (the K split
// is grid.z alone), so the four waves read the same V fragments at about
// the same time (one L2 read, the others from L1) and need no reduction.
template <int NJ, bool ROUTE, bool SH, bool WT = false>
__global__ void __launch_bounds__(256) lowrank_project_kernel(FfnArgs a, int mode, int njy, RouteOut ro) {
  static_assert(!WT || (!SH && !ROUTE), "wave tiles: mode 1 without shared factors");
  __shared__ f32x4 s_part[4][NJ][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (mode != 1 && (int)blockIdx.y >= njy) {
    if constexpr (ROUTE) {
      if ((int)blockIdx.y > njy) {
        if (blockIdx.x == 0 && blockIdx.z == 0) {
          __shared__ RouteLds<4> s_route;
          route_block<256>(ro, a.T, a.E, a.k, s_route);
        }
        return;
      }
    }
    xexp_rows(a, ((int)blockIdx.z * (int)gridDim.x + (int)blockIdx.x) * 4 + wave, (int)(gridDim.x * gridDim.z) * 4);
    return;
  }
  // mode 2: every (token, expert) pair, tokens in place of sorted positions
  const bool tok = mode == 2;
  Chunk ch;
  int sub;
  if (tok) {
    ch.e = (int)blockIdx.x % a.E;
    sub = (int)blockIdx.x / a.E;
    ch.m0 = 0; ch.base = 0; ch.cnt = a.T;
  } else if (WT) {
    sub = wave;
    if (!find_chunk<64>(a.offsets, a.E, blockIdx.x, &ch)) return;
  } else {
    sub = blockIdx.x % kSubPerChunk;
    if (!find_chunk(a.offsets, a.E, blockIdx.x / kSubPerChunk, &ch)) return;
  }
  // (with WT a wave past the chunk's end leaves alone: no barrier follows)
  if (16 * sub >= ch.cnt) return;
  // the tile's pairs (rows past the count repeat the last one)
  const int mloc = std::min(16 * sub + (lane & 15), ch.cnt - 1);
  const int pos = ch.base + mloc;
  // by sorted position: a pair outside its token's leading n_comp slots
  // gets a zero row; by token (mode 2) the consumer applies that mask
  const bool comp_row = tok || (a.sorted_pairs[pos] % a.k) < a.n_comp;
  const bool tile_comp = __ballot(comp_row) != 0;   // the same in every wave of the tile
  const bool gu = mode != 1;
  // shared factors (see slot_group): the group of the lane's row — its
  // member mask, whether the row leads it and (mode 1) the leader's
  // position and the row's factor f.  The token's first eight slots are
  // requested now (with the row's own gate and h exponent), folded after
  // the main loop and handed to the store phase through LDS.  Gate/up:
  // V_G x is computed for every row of a tile; only the leader of each
  // (token, group) stores it, into the rows of all members (mode 2: the
  // group's first expert, for the group's experts).
  const bool grp = SH && !tok && comp_row;
  SlotBatch sb;
  float g_own = 0.f;
  int eh_own = 0, p_own = 0;
  if (grp) {
    p_own = a.sorted_pairs[pos];
    if (gu) {
      slot_batch_load<false>(a, (int64_t)(p_own / a.k) * a.k, 0, sb);
    } else {
      slot_batch_load<true>(a, (int64_t)(p_own / a.k) * a.k, 0, sb);
      g_own = a.gates[p_own];
      eh_own = a.hexpf[p_own];
    }
  }
  // mode 1: y slice 0 writes hn
  const bool write_hn = mode == 1 && blockIdx.y == 0;
  const int jobs_per_blk = (a.Rp + a.Rsp) / 16;
  const int K = gu ? a.H : a.I;
  const int KS = gu ? a.ks_gu : a.ks_d;
  float *zbase = gu ? a.zp_gu + blockIdx.z * a.ks_stride_gu : a.zp_d + blockIdx.z * a.ks_stride_d;
  const int zstride = gu ? 2 * a.RZ : a.RZ;
  // output row of chunk row m: its sorted position, or (mode 2) token * E + e
  auto zrow = [&](int m) -> int64_t { return tok ? (int64_t)m * a.E + ch.e : (int64_t)(ch.base + m); };
  int zcol[NJ];
  bool live[NJ], vi[NJ], shj[NJ];
  const uint16_t *vrow[NJ];
  bool any = false;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int job = (int)blockIdx.y * NJ + j;
    const int bi = job / jobs_per_blk, rem = job % jobs_per_blk;
    const int set = rem < a.Rp / 16 ? 0 : 1;
    const int it = set ? rem - a.Rp / 16 : rem;
    const BlockDesc &d = a.desc[3 * ch.e + (gu ? bi : 2)];
    const uint16_t *V = set ? d.Vs : d.V;
    const int R = set ? a.rs : a.r;
    zcol[j] = bi * a.RZ + set * a.Rp + 16 * it + (lane & 15);
    // a job wholly in the rank padding (rank 8 or 16 padded to 32) loads
    // nothing and writes zero rows
    shj[j] = gu && set == 1;
    live[j] = 16 * it < R;
    any = any || live[j];
    const int i = 16 * it + (lane & 15);
    vi[j] = live[j] && i < R;
    vrow[j] = V + (int64_t)std::min(i, R - 1) * K + 8 * (lane >> 4);
  }
  // zero z rows for the tile (by wave 0; shared columns are written by the
  // groups' leaders, and their readers mask uncompensated pairs)
  auto zero_rows = [&]() {
    if (WT || wave == 0)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = 16 * sub + 4 * (lane >> 4) + q;
        if (m < ch.cnt)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            if (!shj[j] && !(mode == 1 && zcol[j] >= a.Rp)) zbase[zrow(m) * zstride + zcol[j]] = 0.0f;
      }
  };
  // (y slice 0 always holds a live job in mode 1: rank tile 0 of the first
  // factor set with a nonzero rank, so the workgroups that store hn never
  // exit here)
  if (!any) {
    zero_rows();
    return;
  }
  const uint16_t *arow = mode == 0 ? a.x + (int64_t)(a.sorted_pairs[pos] / a.k) * a.H
                         : mode == 2 ? a.x + (int64_t)pos * a.H
                                     : a.h + (int64_t)pos * a.I;
  arow += 8 * (lane >> 4);
  // mode 1: the lane's row of h is renormalised per 64-column block by
  // 2^(eb - eh) (32-column steps st lie in block st / 2); y slice 0 stores
  // the result for the rows of the chunk
  const int eh = mode == 1 ? a.hexp[pos] : 0;
  const int8_t *ebrow = a.hblk + (int64_t)pos * a.hblk_stride;
  uint16_t *hnrow = a.hn + (int64_t)pos * a.I + 8 * (lane >> 4);
  const bool store_hn = write_hn && 16 * sub + (lane & 15) < ch.cnt;
  // mode 1: h fragment of step st (block exponent eb) renormalised to eh
  // (and stored by slice 0)
  auto renorm = [&](f16x8 v, int st, int eb) -> f16x8 {
    const u32x4 w = scale_f16x8(__builtin_bit_cast(u32x4, v), f16x2_pow2(eb - eh));
    if (store_hn) *reinterpret_cast<u32x4 *>(hnrow + 32 * st) = w;
    return __builtin_bit_cast(f16x8, w);
  };
  const int nsteps = K / 32;
  const int z0 = (int)((int64_t)nsteps * blockIdx.z / KS), z1 = (int)((int64_t)nsteps * (blockIdx.z + 1) / KS);
  const int s0 = WT ? z0 : z0 + (z1 - z0) * wave / 4, s1 = WT ? z1 : z0 + (z1 - z0) * (wave + 1) / 4;
  // no pair of the tile compensated (router-guided top-n): zero z rows, no
  // V loads; in mode 1 slice 0 still stores the tile's renormalised h
  if (!tile_comp) {
    zero_rows();
    if (write_hn) {
      int st = s0;
      for (; st + 8 <= s1; st += 8) {
        f16x8 v[8];
        int e[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          v[u] = load_a(arow + 32 * (st + u));
          e[u] = ebrow[(st + u) >> 1];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) (void)renorm(v[u], st + u, e[u]);
      }
      for (; st < s1; ++st) (void)renorm(load_a(arow + 32 * st), st, ebrow[st >> 1]);
    }
    return;
  }
  // batches of BATCH steps: all their fragment loads are issued before the
  // first MFMA, so each batch waits for memory once
  constexpr int BATCH = NJ >= 8 ? 2 : 8 / NJ;
  const f16x8 zero = pack_b(0, 0, 0, 0);
  f32x4 acc[NJ], acc2[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) { acc[j] = f32x4{0.f, 0.f, 0.f, 0.f}; acc2[j] = acc[j]; }
  int st = s0;
  for (; st + BATCH <= s1; st += BATCH) {
    f16x8 av[BATCH], bv[BATCH][NJ];
    int eb[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      av[u] = load_a(arow + 32 * (st + u));
      // (the block exponents are loaded with the fragments: a byte load
      // after the first hn store would have to wait for it)
      if (mode == 1) eb[u] = ebrow[(st + u) >> 1];
#pragma unroll
      for (int j = 0; j < NJ; ++j) bv[u][j] = vi[j] ? load_a(vrow[j] + 32 * (st + u)) : zero;
    }
    if (mode == 1)
#pragma unroll
      for (int u = 0; u < BATCH; ++u) av[u] = renorm(av[u], st + u, eb[u]);
#pragma unroll
    for (int u = 0; u < BATCH; u += 2)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        acc[j] = mfma16(av[u], bv[u][j], acc[j]);
        acc2[j] = mfma16(av[u + 1], bv[u + 1][j], acc2[j]);
      }
  }
  for (; st < s1; ++st) {
    f16x8 av = load_a(arow + 32 * st);
    if (mode == 1) av = renorm(av, st, ebrow[st >> 1]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = mfma16(av, vi[j] ? load_a(vrow[j] + 32 * st) : zero, acc[j]);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[j][q] += acc2[j][q];
  }
  if constexpr (WT) {
    // the wave's own rows, no reduction
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = 16 * sub + 4 * (lane >> 4) + q;
      if (m < ch.cnt) {
        const bool comp = (a.sorted_pairs[ch.base + m] % a.k) < a.n_comp;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          if (zcol[j] < a.Rp) zbase[zrow(m) * zstride + zcol[j]] = (comp && live[j]) ? acc[j][q] : 0.0f;
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) s_part[wave][j][lane] = acc[j];
  __shared__ int s_grp[16][4];
  if (wave == 0 && lane < 16) {
    int gmask = 0, glead = 0, gpos = 0;
    float gf = 0.f;
    if (grp) {
      const int t = p_own / a.k, j = p_own % a.k;
      if (gu) {
        const SlotGroup sg = slot_group_from<false>(a, t, ch.e / a.share, sb);
        gmask = (int)sg.mask;
        glead = sg.lead == j;
      } else {
        const SlotGroup sg = slot_group_from<true>(a, t, ch.e / a.share, sb);
        gmask = (int)sg.mask;
        glead = sg.lead == j;
        gpos = sg.lead_pos;
        gf = down_factor(down_key(g_own, eh_own), sg.key);
      }
    }
    s_grp[lane][0] = gmask;
    s_grp[lane][1] = glead;
    s_grp[lane][2] = gpos;
    s_grp[lane][3] = __builtin_bit_cast(int, gf);
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    f32x4 sum = s_part[0][j][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 p = s_part[w][j][lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) sum[q] += p[q];
    }
    acc[j] = sum;
  }
  // does this workgroup hold shared jobs (mode 1: the first one writes the
  // leader masks)
  bool any_sh = false, dl_writer = false;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const bool sh1 = mode == 1 && zcol[j] >= a.Rp;
    any_sh = any_sh || shj[j] || sh1;
    if (sh1 && zcol[j] - (lane & 15) == a.Rp && blockIdx.z == 0) dl_writer = true;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = 16 * sub + 4 * (lane >> 4) + q;
    if (m < ch.cnt) {
      // (mode 2 runs beside the routing: it reads no routing array)
      const int p = tok ? 0 : a.sorted_pairs[ch.base + m];
      const bool comp = tok || (p % a.k) < a.n_comp;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (!shj[j] && !(mode == 1 && zcol[j] >= a.Rp))
          zbase[zrow(m) * zstride + zcol[j]] = (comp && live[j]) ? acc[j][q] : 0.0f;
      if (!any_sh || !comp || (!SH && !tok)) continue;
      const int r = m - 16 * sub;
      if (gu) {
        // the leader writes V_G x into the row of every member of its group
        if (tok) {
          if (ch.e % a.share != 0) continue;
          for (int e2 = ch.e; e2 < std::min(a.E, ch.e + a.share); ++e2)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              if (shj[j]) zbase[((int64_t)m * a.E + e2) * zstride + zcol[j]] = live[j] ? acc[j][q] : 0.0f;
        } else {
          if (!s_grp[r][1]) continue;
          const int t = p / a.k, js = p % a.k;
          for (uint32_t mask = (uint32_t)s_grp[r][0]; mask; mask &= mask - 1) {
            const int j2 = __builtin_ctz(mask);
            const int64_t r2 = j2 == js ? (int64_t)(ch.base + m) : (int64_t)a.pair_pos[t * a.k + j2];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              if (shj[j]) zbase[r2 * zstride + zcol[j]] = live[j] ? acc[j][q] : 0.0f;
          }
        }
      } else {
        // down: f V_G hn into the member's sub-row of the leader's row; the
        // leader's row also gets the member mask
        const int js = p % a.k;
        const float f = __builtin_bit_cast(float, s_grp[r][3]);
        float *dst = a.zsh + blockIdx.z * a.ks_stride_sh + ((int64_t)s_grp[r][2] * a.k + js) * a.Rsp;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          if (zcol[j] >= a.Rp) dst[zcol[j] - a.Rp] = live[j] ? acc[j][q] * f : 0.0f;
        if (dl_writer && (lane & 15) == 0) a.dlead[ch.base + m] = s_grp[r][1] ? s_grp[r][0] : 0;
      }
    }
  }
}

// y[t] = sum_j g[t][j] * 2^(eh - kNormTop) * sum_s ypart[s][pair_pos[t*k+j]],
// slots in order, splits in order within a slot; one thread per (token, 4
// columns); eh is the h exponent of the pair (see hexp).  Slots
// go in groups of 4: their gates and positions are loaded together, then
// every partial of the group (up to MS splits each; MS = 1 when there is
// one split, so that the many-token case keeps few registers) is requested
// before the first add, so a group costs two memory round trips, not one
// per partial.
template <bool F32, int MS>
__global__ void __launch_bounds__(256) combine_kernel(FfnArgs a, void *y) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_t = a.H / 4;
  if (id >= (int64_t)a.T * per_t) return;
  const int t = (int)(id / per_t), c = (int)(id % per_t) * 4;
  const int64_t tk = (int64_t)t * a.k;
  const int ns = a.splits;
  f32x4 out = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < a.k; j0 += 4) {
    float g[4];
    int pos[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const bool ok = j0 + jj < a.k;
      pos[jj] = ok ? a.pair_pos[tk + j0 + jj] : 0;
      // y_pair is held in units of 2^(eh - kNormTop) of its pair
      g[jj] = ok ? __builtin_ldexpf(a.gates[tk + j0 + jj], a.hexp[pos[jj]] - kNormTop) : 0.f;
    }
    f32x4 v[4][MS];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int s = 0; s < MS; ++s)
        if (j0 + jj < a.k && s < ns)
          v[jj][s] = *reinterpret_cast<const f32x4 *>(a.ypart + ((int64_t)s * a.P + pos[jj]) * a.H + c);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (j0 + jj >= a.k) break;
      f32x4 sum = v[jj][0];
#pragma unroll
      for (int s = 1; s < MS; ++s)
        if (s < ns)
#pragma unroll
          for (int q = 0; q < 4; ++q) sum[q] += v[jj][s][q];
      for (int s = MS; s < ns; ++s) {
        const f32x4 p = *reinterpret_cast<const f32x4 *>(a.ypart + ((int64_t)s * a.P + pos[jj]) * a.H + c);
#pragma unroll
        for (int q = 0; q < 4; ++q) sum[q] += p[q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) out[q] = __builtin_fmaf(g[jj], sum[q], out[q]);
    }
  }
  if (F32) {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(y) + (int64_t)t * a.H + c) = out;
  } else {
    uint16_t *yo = static_cast<uint16_t *>(y) + (int64_t)t * a.H + c;
    u32x2 w;
    w[0] = as_u32(f16x2{(f16)out[0], (f16)out[1]});
    w[1] = as_u32(f16x2{(f16)out[2], (f16)out[3]});
    *reinterpret_cast<u32x2 *>(yo) = w;
  }
}

void launch_lowrank_project(const FfnArgs &a, int mode, int jobs, hipStream_t s) {
  if (mode == 1 && a.wt) {
    // wave tiles: all jobs of a 64-pair chunk in one workgroup
    const dim3 grid(max_chunks(a.E, a.T, a.k, 64), 1, a.ks_d);
    const RouteOut ro{};
    switch (jobs) {
      case 4: hipLaunchKernelGGL((lowrank_project_kernel<4, false, false, true>), grid, dim3(256), 0, s, a, 1, 1, ro); break;
      case 2: hipLaunchKernelGGL((lowrank_project_kernel<2, false, false, true>), grid, dim3(256), 0, s, a, 1, 1, ro); break;
      default: hipLaunchKernelGGL((lowrank_project_kernel<1, false, false, true>), grid, dim3(256), 0, s, a, 1, 1, ro); break;
    }
    return;
  }
  dim3 grid(mode == 2 ? (a.T + 15) / 16 * a.E : max_chunks(a.E, a.T, a.k) * kSubPerChunk, jobs,
            mode != 1 ? a.ks_gu : a.ks_d);
  // two, four or eight jobs per workgroup when many tokens leave no K
  // split (the activation re-reads dominate; fewer jobs keep enough
  // workgroups); the job count is always even.  Four jobs in one workgroup
  // when there are just four: on the down side only (bit-plane layer with
  // rank 8 + shared 32: 24.6 -> 23.5 us at 512 tokens, 101 -> 72 us at
  // 4096; on the gate/up side the fine-grained layer's projection went
  // from 16.0 to 17.5 us)
  int nj = 1;
  if (a.P > 256 && grid.z == 1 && grid.y % 8 == 0) nj = 8;
  else if (a.P > 256 && grid.z == 1 && grid.y % 4 == 0 && (grid.y >= 8 || mode == 1)) nj = 4;
  else if (a.P > 256 && grid.z == 1 && grid.y % 2 == 0) nj = 2;
  grid.y /= nj;
  const int njy = (int)grid.y;
  if (mode != 1) grid.y += 1;                 // the x-exponent slice
  const RouteOut ro{};
  if (a.rs > 0) {
    switch (nj) {
      case 8: hipLaunchKernelGGL((lowrank_project_kernel<8, false, true>), grid, dim3(256), 0, s, a, mode, njy, ro); break;
      case 4: hipLaunchKernelGGL((lowrank_project_kernel<4, false, true>), grid, dim3(256), 0, s, a, mode, njy, ro); break;
      case 2: hipLaunchKernelGGL((lowrank_project_kernel<2, false, true>), grid, dim3(256), 0, s, a, mode, njy, ro); break;
      default: hipLaunchKernelGGL((lowrank_project_kernel<1, false, true>), grid, dim3(256), 0, s, a, mode, njy, ro); break;
    }
  } else {
    switch (nj) {
      case 8: hipLaunchKernelGGL((lowrank_project_kernel<8, false, false>), grid, dim3(256), 0, s, a, mode, njy, ro); break;
      case 4: hipLaunchKernelGGL((lowrank_project_kernel<4, false, false>), grid, dim3(256), 0, s, a, mode, njy, ro); break;
      case 2: hipLaunchKernelGGL((lowrank_project_kernel<2, false, false>), grid, dim3(256), 0, s, a, mode, njy, ro); break;
      default: hipLaunchKernelGGL((lowrank_project_kernel<1, false, false>), grid, dim3(256), 0, s, a, mode, njy, ro); break;
    }
  }
}

// Routing, x exponents and (with compensation) the gate/up projection of
// every (token, expert) pair in one launch; up to kRouteTokens tokens.
// Without compensation there are no projection slices (njy = 0).
void launch_front_routed(const FfnArgs &a, const RouteOut &ro, hipStream_t s) {
  const int njy = a.comp_on ? 2 * a.RZ / 16 : 0;
  const dim3 grid(a.comp_on ? (a.T + 15) / 16 * a.E : (a.T + 3) / 4, njy + 2, a.comp_on ? a.ks_gu : 1);
  // (mode 2 stores shared columns without the group bookkeeping)
  hipLaunchKernelGGL((lowrank_project_kernel<1, true, false>), grid, dim3(256), 0, s, a, 2, njy, ro);
}

// x exponents when no gate/up projection runs: one wave per token.
__global__ void __launch_bounds__(256) xexp_kernel(FfnArgs a) {
  xexp_rows(a, (int)blockIdx.x * 4 + (threadIdx.x >> 6), (int)gridDim.x * 4);
}

// hn when no down projection runs: 16 pairs (sorted positions) per
// workgroup; each thread rescales 16-byte pieces of the rows.
__global__ void __launch_bounds__(256) hnorm_kernel(FfnArgs a) {
  const int pos0 = (int)blockIdx.x * 16;
  const int per_row = a.I / 8;
  for (int i = threadIdx.x; i < 16 * per_row; i += 256) {
    const int r = i / per_row, c = (i % per_row) * 8;
    const int pos = pos0 + r;
    if (pos >= a.P) break;
    const int64_t off = (int64_t)pos * a.I + c;
    const int eb = gld<int8_t>(a.hblk + (int64_t)pos * a.hblk_stride + c / 64);
    *reinterpret_cast<u32x4 *>(a.hn + off) = scale_f16x8(gld<u32x4>(a.h + off), f16x2_pow2(eb - a.hexp[pos]));
  }
}

void launch_xexp(const FfnArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(xexp_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
}

void launch_hnorm(const FfnArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(hnorm_kernel, dim3((a.P + 15) / 16), dim3(256), 0, s, a);
}

void launch_combine(const FfnArgs &a, void *y, bool f32, hipStream_t s) {
  const int64_t n = (int64_t)a.T * (a.H / 4);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (a.splits == 1) {
    if (f32) hipLaunchKernelGGL((combine_kernel<true, 1>), dim3(blocks), dim3(256), 0, s, a, y);
    else hipLaunchKernelGGL((combine_kernel<false, 1>), dim3(blocks), dim3(256), 0, s, a, y);
  } else {
    if (f32) hipLaunchKernelGGL((combine_kernel<true, 4>), dim3(blocks), dim3(256), 0, s, a, y);
    else hipLaunchKernelGGL((combine_kernel<false, 4>), dim3(blocks), dim3(256), 0, s, a, y);
  }
}

}  // namespace moeq
