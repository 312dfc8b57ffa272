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
// One 16-token tile per workgroup, 4 waves split the range and reduce
// through LDS in fixed order.
// grid.x = max_chunks * 4 tiles, grid.y = (#blocks) * (Rp + Rsp) / 16,
// grid.z = ks.  mode 0: v = x[token] (gate/up blocks); mode 1: v = h[pos]
// (down block).
__global__ void __launch_bounds__(256) lowrank_project_kernel(FfnArgs a, int mode) {
  __shared__ f32x4 s_part[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x / 4, sub = blockIdx.x % 4;
  Chunk ch;
  if (!find_chunk(a.offsets, a.E, chunk, &ch)) return;
  if (16 * sub >= ch.cnt) return;
  const int jobs_per_blk = (a.Rp + a.Rsp) / 16;
  const int bi = blockIdx.y / jobs_per_blk, rem = blockIdx.y % jobs_per_blk;
  const int set = rem < a.Rp / 16 ? 0 : 1;
  const int it = set ? rem - a.Rp / 16 : rem;
  const int blk = mode == 0 ? bi : 2;
  const BlockDesc &d = a.desc[3 * ch.e + blk];
  const uint16_t *V = set ? d.Vs : d.V;
  const int R = set ? a.rs : a.r;
  const int K = d.K;
  const int KS = mode == 0 ? a.ks_gu : a.ks_d;
  float *zbase = mode == 0 ? a.zp_gu + blockIdx.z * a.ks_stride_gu : a.zp_d + blockIdx.z * a.ks_stride_d;
  const int zstride = mode == 0 ? 2 * a.RZ : a.RZ;
  const int zcol = bi * a.RZ + set * a.Rp + 16 * it + (lane & 15);
  if (16 * it >= R) {
    // the whole tile is padding past the factor's rank: zero rows, no loads
    if (wave == 0)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = 16 * sub + 4 * (lane >> 4) + q;
        if (m < ch.cnt) zbase[(int64_t)(ch.base + m) * zstride + zcol] = 0.0f;
      }
    return;
  }
  const int i = 16 * it + (lane & 15);
  const int mloc = std::min(16 * sub + (lane & 15), ch.cnt - 1);
  const int pos = ch.base + mloc;
  const uint16_t *arow = (mode == 0) ? a.x + (int64_t)(a.sorted_pairs[pos] / a.k) * a.H
                                     : a.h + (int64_t)pos * a.I;
  arow += 8 * (lane >> 4);
  const uint16_t *vrow = V + (int64_t)std::min(i, R - 1) * K + 8 * (lane >> 4);
  const bool vi = i < R;
  const int nsteps = K / 32;
  const int z0 = (int)((int64_t)nsteps * blockIdx.z / KS), z1 = (int)((int64_t)nsteps * (blockIdx.z + 1) / KS);
  const int s0 = z0 + (z1 - z0) * wave / 4, s1 = z0 + (z1 - z0) * (wave + 1) / 4;
  // batches of 8 steps: all 16 fragment loads are issued before the first
  // MFMA, so each batch waits for memory once
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = acc;
  int st = s0;
  for (; st + 8 <= s1; st += 8) {
    f16x8 av[8], bv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      av[u] = load_a(arow + 32 * (st + u));
      bv[u] = vi ? load_a(vrow + 32 * (st + u)) : pack_b(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      acc = mfma16(av[u], bv[u], acc);
      acc2 = mfma16(av[u + 1], bv[u + 1], acc2);
    }
  }
  for (; st < s1; ++st) {
    const f16x8 b = vi ? load_a(vrow + 32 * st) : pack_b(0, 0, 0, 0);
    acc = mfma16(load_a(arow + 32 * st), b, acc);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] += acc2[q];
  s_part[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 sum = s_part[0][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const f32x4 p = s_part[w][lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) sum[q] += p[q];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = 16 * sub + 4 * (lane >> 4) + q;
    if (m < ch.cnt) {
      const int p2 = ch.base + m;
      const bool comp = (a.sorted_pairs[p2] % a.k) < a.n_comp;
      zbase[(int64_t)p2 * zstride + zcol] = comp ? sum[q] : 0.0f;
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
  hipLaunchKernelGGL(lowrank_project_kernel, grid, dim3(256), 0, s, a, mode);
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
