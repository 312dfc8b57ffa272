// Skinny low-rank projections and the gate-weighted combine.
//
// z = V v for each compensated pair (MiLo abstract: low-rank compensators;
// TileQ abstract: factors shared by a group of experts, so each pair also
// gets the group's V_G v; Bandwidth-Efficient Adaptive MoE abstract: only a
// token's top-n slots are compensated, the other rows of z are zero), and
// y_t = sum_j g_{t,j} y_pair(t, j) summed in slot order.
#include "common.hpp"
#include "ffn.hpp"

namespace moeq {

// Partial z[pos][slot] = V v over one K range for compensated pairs (zero
// for the others); the consumer kernels sum the ks partials in fixed order.
// One 16-token tile and NJ 16-column jobs per workgroup (NJ = 2, 4 or 8
// when many tokens leave no K split: each activation fragment then feeds
// every job, so the activations are read NJ times less often); 4 waves
// split the range and reduce through LDS in fixed order.
// grid.x = max_chunks * kSubPerChunk tiles, grid.y = (#blocks) * (Rp + Rsp) / 16 / NJ,
// grid.z = ks.  mode 0: v = x[token] (gate/up blocks); mode 1: v = h[pos]
// (down block).
template <int NJ>
__global__ void __launch_bounds__(256) lowrank_project_kernel(FfnArgs a, int mode) {
  __shared__ f32x4 s_part[4][NJ][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x / kSubPerChunk, sub = blockIdx.x % kSubPerChunk;
  Chunk ch;
  if (!find_chunk(a.offsets, a.E, chunk, &ch)) return;
  if (16 * sub >= ch.cnt) return;
  const int jobs_per_blk = (a.Rp + a.Rsp) / 16;
  const int K = mode == 0 ? a.H : a.I;
  const int KS = mode == 0 ? a.ks_gu : a.ks_d;
  float *zbase = mode == 0 ? a.zp_gu + blockIdx.z * a.ks_stride_gu : a.zp_d + blockIdx.z * a.ks_stride_d;
  const int zstride = mode == 0 ? 2 * a.RZ : a.RZ;
  int zcol[NJ];
  bool live[NJ], vi[NJ];
  const uint16_t *vrow[NJ];
  bool any = false;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int job = (int)blockIdx.y * NJ + j;
    const int bi = job / jobs_per_blk, rem = job % jobs_per_blk;
    const int set = rem < a.Rp / 16 ? 0 : 1;
    const int it = set ? rem - a.Rp / 16 : rem;
    const BlockDesc &d = a.desc[3 * ch.e + (mode == 0 ? bi : 2)];
    const uint16_t *V = set ? d.Vs : d.V;
    const int R = set ? a.rs : a.r;
    zcol[j] = bi * a.RZ + set * a.Rp + 16 * it + (lane & 15);
    // a job wholly in the rank padding (rank 8 or 16 padded to 32) loads
    // nothing and writes zero rows
    live[j] = 16 * it < R;
    any = any || live[j];
    const int i = 16 * it + (lane & 15);
    vi[j] = live[j] && i < R;
    vrow[j] = V + (int64_t)std::min(i, R - 1) * K + 8 * (lane >> 4);
  }
  if (!any) {
    if (wave == 0)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = 16 * sub + 4 * (lane >> 4) + q;
        if (m < ch.cnt)
#pragma unroll
          for (int j = 0; j < NJ; ++j) zbase[(int64_t)(ch.base + m) * zstride + zcol[j]] = 0.0f;
      }
    return;
  }
  const int mloc = std::min(16 * sub + (lane & 15), ch.cnt - 1);
  const int pos = ch.base + mloc;
  const uint16_t *arow = (mode == 0) ? a.x + (int64_t)(a.sorted_pairs[pos] / a.k) * a.H
                                     : a.h + (int64_t)pos * a.I;
  arow += 8 * (lane >> 4);
  const int nsteps = K / 32;
  const int z0 = (int)((int64_t)nsteps * blockIdx.z / KS), z1 = (int)((int64_t)nsteps * (blockIdx.z + 1) / KS);
  const int s0 = z0 + (z1 - z0) * wave / 4, s1 = z0 + (z1 - z0) * (wave + 1) / 4;
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
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      av[u] = load_a(arow + 32 * (st + u));
#pragma unroll
      for (int j = 0; j < NJ; ++j) bv[u][j] = vi[j] ? load_a(vrow[j] + 32 * (st + u)) : zero;
    }
#pragma unroll
    for (int u = 0; u < BATCH; u += 2)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        acc[j] = mfma16(av[u], bv[u][j], acc[j]);
        acc2[j] = mfma16(av[u + 1], bv[u + 1][j], acc2[j]);
      }
  }
  for (; st < s1; ++st) {
    const f16x8 av = load_a(arow + 32 * st);
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = mfma16(av, vi[j] ? load_a(vrow[j] + 32 * st) : zero, acc[j]);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[j][q] += acc2[j][q];
    s_part[wave][j][lane] = acc[j];
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
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = 16 * sub + 4 * (lane >> 4) + q;
    if (m < ch.cnt) {
      const int p2 = ch.base + m;
      const bool comp = (a.sorted_pairs[p2] % a.k) < a.n_comp;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        zbase[(int64_t)p2 * zstride + zcol[j]] = (comp && live[j]) ? acc[j][q] : 0.0f;
    }
  }
}

// y[t] = sum_j g[t][j] * sum_s ypart[s][pair_pos[t*k+j]], slots in order,
// splits in order within a slot; one thread per (token, 4 columns).  Slots
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
      g[jj] = ok ? a.gates[tk + j0 + jj] : 0.f;
      pos[jj] = ok ? a.pair_pos[tk + j0 + jj] : 0;
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

void launch_lowrank_project(const FfnArgs &a, int mode, dim3 grid, hipStream_t s) {
  grid.z = mode == 0 ? a.ks_gu : a.ks_d;
  // two, four or eight jobs per workgroup when many tokens leave no K
  // split (the activation re-reads dominate; fewer jobs keep enough
  // workgroups); the job count is always even
  if (a.P > 256 && grid.z == 1 && grid.y % 8 == 0) {
    grid.y /= 8;
    hipLaunchKernelGGL(lowrank_project_kernel<8>, grid, dim3(256), 0, s, a, mode);
  } else if (a.P > 256 && grid.z == 1 && grid.y % 4 == 0 && grid.y >= 8) {
    grid.y /= 4;
    hipLaunchKernelGGL(lowrank_project_kernel<4>, grid, dim3(256), 0, s, a, mode);
  } else if (a.P > 256 && grid.z == 1 && grid.y % 2 == 0) {
    grid.y /= 2;
    hipLaunchKernelGGL(lowrank_project_kernel<2>, grid, dim3(256), 0, s, a, mode);
  } else {
    hipLaunchKernelGGL(lowrank_project_kernel<1>, grid, dim3(256), 0, s, a, mode);
  }
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
