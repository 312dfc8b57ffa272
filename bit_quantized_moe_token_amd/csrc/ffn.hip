// Routed expert FFN on packed low-bit weights (weight-streaming path).
//
//   a = L_gate(x), b = L_up(x), h = SiLU(a) * b, y_pair = L_down(h),
//   L(v) = W_hat v + comp * (U (V v) + U_G (V_G v)),
//   y_t = sum_j g_{t,j} y_pair(t, j)
//
// Sources: MiLo abstract (low-rank compensators on extreme-low-bit experts),
// TileQ abstract (factors shared across experts; low-rank terms fused into
// the expert pass), Bandwidth-Efficient Adaptive MoE abstract (only the
// top-n slots of a token are compensated), PagedWeight review summary (one
// fused kernel executing variable bitwidths), MxMoE abstract (per-block
// bitwidths, uneven expert activation).
//
// Work decomposition.  The tokens routed to one expert are cut into chunks
// of up to 64 (four 16-row MFMA tiles).  A wave owns one 16-row strip of a
// weight block for one chunk and streams the strip once over K: per
// 128-column tile it loads its 32 packed codes with 128-bit loads, decodes
// them in registers into fp16 (c - z) pairs (INT) or LUT values (bit-plane)
// and feeds v_mfma_f32_16x16x32_f16 with the chunk's activations as the A
// operand.  INT blocks accumulate per quantization group and apply the fp16
// scale to the fp32 group sum.  The low-rank term is one more MFMA in the
// epilogue (A = z = V v from a small projection kernel, B = U^T).
//
// Kernels per call: project V x (gate/up), gate/up + SwiGLU -> h,
// project V_down h, down (split-K) -> y_pair partials, combine.
#include <algorithm>
#include "common.hpp"
#include "decode.hpp"
#include "layer.hpp"

namespace moeq {

constexpr int kMT = 64;            // tokens per chunk
constexpr int kSub = kMT / 16;     // MFMA row tiles per chunk
constexpr int kStripsPerWG = 4;    // one strip per wave

struct Chunk {
  int e, m0, cnt, base;
};

// Chunk c of the expert-major chunk list: expert e, first token m0 within
// the expert, token count, and first sorted position.
__device__ __forceinline__ bool find_chunk(const int32_t *__restrict__ off, int E, int c, Chunk *out) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int b = 0; b < E; b += kWave) {
    const int e = b + lane;
    const int cnt = e < E ? off[e + 1] - off[e] : 0;
    const int nc = (cnt + kMT - 1) / kMT;
    int incl = nc;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += t;
    }
    const int excl = carry + incl - nc;
    const uint64_t hit = __ballot(c >= excl && c < excl + nc);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      const int ex = __shfl(excl, src, kWave);
      const int cn = __shfl(cnt, src, kWave);
      out->e = b + src;
      out->m0 = (c - ex) * kMT;
      out->cnt = std::min(kMT, cn - out->m0);
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

__device__ __forceinline__ f16x8 pack_b(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(f16x8, v);
}

// Lane words of a tile group: C tiles of W4 dwords each.
template <int N, bool VEC>
__device__ __forceinline__ void load_words(const uint8_t *p, uint32_t *w) {
  if (VEC) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const u32x4 v = reinterpret_cast<const u32x4 *>(p)[i];
      w[4 * i] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = reinterpret_cast<const uint32_t *>(p)[i];
  }
}

// ----------------------------------------------------------------- INT --
// Streams tiles [g4_begin*4, g4_end*4) of one strip of a B-bit block.
// acc[s] accumulates token tile s (16 rows of the chunk).
template <int B, int GPT, int C>
__device__ __forceinline__ void int_group(const BlockDesc &d, int strip, int g4, int n_kt,
                                          const uint16_t *const *arow, int nsub, f32x4 *acc) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  uint32_t cw[C * B];
  load_words<C * B, C == 4>(d.codes + code_offset(strip, 4 * g4, lane, n_kt, 4 * B), cw);
  const uint64_t mi = meta_index(strip, 4 * g4, r, 0, n_kt, GPT);
  uint16_t sc[C * GPT];
  uint8_t zz[C * GPT];
#pragma unroll
  for (int i = 0; i < C * GPT; ++i) { sc[i] = d.scales[mi + i]; zz[i] = d.zeros[mi + i]; }
#pragma unroll
  for (int tl = 0; tl < C; ++tl) {
    const int t = 4 * g4 + tl;
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      PairConst pc[9];
      fill_pair_consts<B>(pc, (float)zz[tl * GPT + gi]);
      f32x4 part[kSub];
#pragma unroll
      for (int s = 0; s < kSub; ++s) part[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 4 / GPT; ++jj) {
        const int j = gi * (4 / GPT) + jj;
        const uint32_t *dw = cw + tl * B;
        const f16x8 bop = pack_b(int_pair_cz<B>(dw, 4 * j + 0, pc), int_pair_cz<B>(dw, 4 * j + 1, pc),
                                 int_pair_cz<B>(dw, 4 * j + 2, pc), int_pair_cz<B>(dw, 4 * j + 3, pc));
#pragma unroll
        for (int s = 0; s < kSub; ++s)
          if (s < nsub) part[s] = mfma16(load_a(arow[s] + t * kTileK + 32 * j), bop, part[s]);
      }
      const float scale = (float)__builtin_bit_cast(f16, sc[tl * GPT + gi]);
#pragma unroll
      for (int s = 0; s < kSub; ++s)
        if (s < nsub) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[s][i] = __builtin_fmaf(scale, part[s][i], acc[s][i]);
        }
    }
  }
}

template <int B, int GPT>
__device__ __forceinline__ void int_strip(const BlockDesc &d, int strip, int g4_begin, int g4_end,
                          const uint16_t *const *arow, int nsub, f32x4 *acc) {
  const int n_kt = d.K / kTileK;
  const int full = n_kt / 4;
  const int stop = std::min(g4_end, full);
  for (int g4 = g4_begin; g4 < stop; ++g4) int_group<B, GPT, 4>(d, strip, g4, n_kt, arow, nsub, acc);
  if (g4_end > full && (n_kt & 3)) {
    switch (n_kt & 3) {
      case 1: int_group<B, GPT, 1>(d, strip, full, n_kt, arow, nsub, acc); break;
      case 2: int_group<B, GPT, 2>(d, strip, full, n_kt, arow, nsub, acc); break;
      default: int_group<B, GPT, 3>(d, strip, full, n_kt, arow, nsub, acc); break;
    }
  }
}

// ----------------------------------------------------------- bit-plane --
template <int Q, int C>
__device__ __forceinline__ void plane_group(const BlockDesc &d, int strip, int g4, int n_kt,
                                            const uint16_t *const *arow, int nsub, f32x4 *acc) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  constexpr int NQ = 1 << Q;
  const uint64_t off = code_offset(strip, 4 * g4, lane, n_kt, 4);
  uint32_t pl[Q][C];
#pragma unroll
  for (int u = 0; u < Q; ++u) load_words<C, C == 4>(d.codes + u * d.plane_bytes + off, pl[u]);
#pragma unroll
  for (int tl = 0; tl < C; ++tl) {
    const int t = 4 * g4 + tl;
    uint32_t L[NQ / 2];
    const uint32_t *lp = reinterpret_cast<const uint32_t *>(d.lut + lut_index(strip, t, r, 0, n_kt, NQ));
#pragma unroll
    for (int i = 0; i < NQ / 2; ++i) L[i] = lp[i];
    uint32_t tp[Q];
#pragma unroll
    for (int u = 0; u < Q; ++u) tp[u] = pl[u][tl];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t m = plane_merge<Q>(tp, j);
      uint32_t pr[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) pr[v] = lut_pair<Q>((m >> (4 * v)) & 0x000F000Fu, L);
      const f16x8 bop = pack_b(pr[0], pr[1], pr[2], pr[3]);
#pragma unroll
      for (int s = 0; s < kSub; ++s)
        if (s < nsub) acc[s] = mfma16(load_a(arow[s] + t * kTileK + 32 * j), bop, acc[s]);
    }
  }
}

template <int Q>
__device__ __forceinline__ void plane_strip(const BlockDesc &d, int strip, int g4_begin, int g4_end,
                            const uint16_t *const *arow, int nsub, f32x4 *acc) {
  const int n_kt = d.K / kTileK;
  const int full = n_kt / 4;
  const int stop = std::min(g4_end, full);
  for (int g4 = g4_begin; g4 < stop; ++g4) plane_group<Q, 4>(d, strip, g4, n_kt, arow, nsub, acc);
  if (g4_end > full && (n_kt & 3)) {
    switch (n_kt & 3) {
      case 1: plane_group<Q, 1>(d, strip, full, n_kt, arow, nsub, acc); break;
      case 2: plane_group<Q, 2>(d, strip, full, n_kt, arow, nsub, acc); break;
      default: plane_group<Q, 3>(d, strip, full, n_kt, arow, nsub, acc); break;
    }
  }
}

// One strip of one block over tile groups [g4_begin, g4_end).
template <int GPT>
__device__ __forceinline__ void run_strip(const BlockDesc &d, int strip, int g4_begin, int g4_end,
                          const uint16_t *const *arow, int nsub, f32x4 *acc) {
  if (d.fmt == MOEQ_FMT_INT) {
    switch (d.bits) {
      case 2: int_strip<2, GPT>(d, strip, g4_begin, g4_end, arow, nsub, acc); break;
      case 3: int_strip<3, GPT>(d, strip, g4_begin, g4_end, arow, nsub, acc); break;
      default: int_strip<4, GPT>(d, strip, g4_begin, g4_end, arow, nsub, acc); break;
    }
  } else {
    switch (d.bits) {
      case 2: plane_strip<2>(d, strip, g4_begin, g4_end, arow, nsub, acc); break;
      case 3: plane_strip<3>(d, strip, g4_begin, g4_end, arow, nsub, acc); break;
      default: plane_strip<4>(d, strip, g4_begin, g4_end, arow, nsub, acc); break;
    }
  }
}

// Low-rank epilogue: acc += U (z) for one factor set; z rows are fp16 with
// zeros for uncompensated pairs and for columns >= R.  zrow[s] already
// points at this lane's 8-column slot (8 * (lane / 16)) of its token's row.
__device__ __forceinline__ void lowrank_epilogue(const uint16_t *U, int R, int Rpad, int row,
                                                 const uint16_t *const *zrow, int nsub, f32x4 *acc) {
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4;
  for (int ks = 0; ks < Rpad / 32; ++ks) {
    const int col = 32 * ks + 8 * kq;
    f16x8 bop = pack_b(0, 0, 0, 0);
    if (col < R) bop = load_a(U + (int64_t)row * R + col);
#pragma unroll
    for (int s = 0; s < kSub; ++s)
      if (s < nsub) acc[s] = mfma16(load_a(zrow[s] + 32 * ks), bop, acc[s]);
  }
}

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
  uint16_t *z_gu;   // [P][2][RZ]
  uint16_t *z_d;    // [P][RZ]
  uint16_t *h;      // [P][I]
  float *ypart;     // [S][P][H]
  int splits;
  int P;
};

// gate/up + SwiGLU.  grid.x = max_chunks * (I / 64); 4 waves = 4 strips.
template <int GPT>
__global__ void __launch_bounds__(256) gateup_stream_kernel(FfnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n_sg = a.I / (16 * kStripsPerWG);
  const int chunk = blockIdx.x / n_sg, sg = blockIdx.x % n_sg;
  Chunk ch;
  if (!find_chunk(a.offsets, a.E, chunk, &ch)) return;
  const int strip = sg * kStripsPerWG + wave;
  const int nsub = (ch.cnt + 15) / 16;
  const uint16_t *arow[kSub];
#pragma unroll
  for (int s = 0; s < kSub; ++s) {
    const int m = std::min(16 * s + (lane & 15), ch.cnt - 1);
    const int tok = a.sorted_pairs[ch.base + m] / a.k;
    arow[s] = a.x + (int64_t)tok * a.H + 8 * (lane >> 4);
  }
  f32x4 accg[kSub], accu[kSub];
#pragma unroll
  for (int s = 0; s < kSub; ++s) { accg[s] = f32x4{0.f, 0.f, 0.f, 0.f}; accu[s] = accg[s]; }
  const BlockDesc dg = a.desc[3 * ch.e], du = a.desc[3 * ch.e + 1];
  const int n_g4 = (dg.K / kTileK + 3) / 4;
  run_strip<GPT>(dg, strip, 0, n_g4, arow, nsub, accg);
  run_strip<GPT>(du, strip, 0, n_g4, arow, nsub, accu);
  const int row = strip * 16 + (lane & 15);
  if (a.comp_on) {
    const uint16_t *zr[kSub];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const BlockDesc &d = blk ? du : dg;
      f32x4 *acc = blk ? accu : accg;
#pragma unroll
      for (int s = 0; s < kSub; ++s) {
        const int m = std::min(16 * s + (lane & 15), ch.cnt - 1);
        zr[s] = a.z_gu + (int64_t)(ch.base + m) * 2 * a.RZ + blk * a.RZ + 8 * (lane >> 4);
      }
      if (a.r > 0) lowrank_epilogue(d.U, a.r, a.Rp, row, zr, nsub, acc);
      if (a.rs > 0) {
#pragma unroll
        for (int s = 0; s < kSub; ++s) zr[s] += a.Rp;
        lowrank_epilogue(d.Us, a.rs, a.Rsp, row, zr, nsub, acc);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < kSub; ++s) {
    if (s >= nsub) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * s + 4 * (lane >> 4) + i;
      if (m < ch.cnt) {
        const float g = accg[s][i], u = accu[s][i];
        const float hv = g / (1.0f + __expf(-g)) * u;
        a.h[(int64_t)(ch.base + m) * a.I + row] = __builtin_bit_cast(uint16_t, (f16)hv);
      }
    }
  }
}

// down projection; grid.x = max_chunks * (H / 64) * splits.
template <int GPT>
__global__ void __launch_bounds__(256) down_stream_kernel(FfnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n_sg = a.H / (16 * kStripsPerWG);
  const int split = blockIdx.x % a.splits;
  const int rest = blockIdx.x / a.splits;
  const int chunk = rest / n_sg, sg = rest % n_sg;
  Chunk ch;
  if (!find_chunk(a.offsets, a.E, chunk, &ch)) return;
  const int strip = sg * kStripsPerWG + wave;
  const int nsub = (ch.cnt + 15) / 16;
  const uint16_t *arow[kSub];
#pragma unroll
  for (int s = 0; s < kSub; ++s) {
    const int m = std::min(16 * s + (lane & 15), ch.cnt - 1);
    arow[s] = a.h + (int64_t)(ch.base + m) * a.I + 8 * (lane >> 4);
  }
  f32x4 acc[kSub];
#pragma unroll
  for (int s = 0; s < kSub; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
  const BlockDesc dd = a.desc[3 * ch.e + 2];
  const int n_g4 = (dd.K / kTileK + 3) / 4;
  const int g0 = (int)((int64_t)n_g4 * split / a.splits);
  const int g1 = (int)((int64_t)n_g4 * (split + 1) / a.splits);
  run_strip<GPT>(dd, strip, g0, g1, arow, nsub, acc);
  const int row = strip * 16 + (lane & 15);
  if (a.comp_on && split == 0) {
    const uint16_t *zr[kSub];
#pragma unroll
    for (int s = 0; s < kSub; ++s) {
      const int m = std::min(16 * s + (lane & 15), ch.cnt - 1);
      zr[s] = a.z_d + (int64_t)(ch.base + m) * a.RZ + 8 * (lane >> 4);
    }
    if (a.r > 0) lowrank_epilogue(dd.U, a.r, a.Rp, row, zr, nsub, acc);
    if (a.rs > 0) {
#pragma unroll
      for (int s = 0; s < kSub; ++s) zr[s] += a.Rp;
      lowrank_epilogue(dd.Us, a.rs, a.Rsp, row, zr, nsub, acc);
    }
  }
  float *yp = a.ypart + (int64_t)split * a.P * a.H;
#pragma unroll
  for (int s = 0; s < kSub; ++s) {
    if (s >= nsub) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * s + 4 * (lane >> 4) + i;
      if (m < ch.cnt) yp[(int64_t)(ch.base + m) * a.H + row] = acc[s][i];
    }
  }
}

// z[pos][slot] = V v for compensated pairs (zero otherwise).  One 16-token
// tile per workgroup, 4 waves split K and reduce through LDS in fixed order.
// grid.x = max_chunks * 4 tiles, grid.y = (#blocks) * (Rp + Rsp) / 16.
// mode 0: v = x[token] (gate/up, blk0 = 0, nblk = 2); mode 1: v = h[pos]
// (down, blk0 = 2, nblk = 1).
__global__ void __launch_bounds__(256) lowrank_project_kernel(FfnArgs a, int mode) {
  __shared__ f32x4 s_part[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x / kSub, sub = blockIdx.x % kSub;
  Chunk ch;
  if (!find_chunk(a.offsets, a.E, chunk, &ch)) return;
  if (16 * sub >= ch.cnt) return;
  const int jobs_per_blk = (a.Rp + a.Rsp) / 16;
  const int bi = blockIdx.y / jobs_per_blk, rem = blockIdx.y % jobs_per_blk;
  const int set = rem < a.Rp / 16 ? 0 : 1;
  const int it = set ? rem - a.Rp / 16 : rem;
  const int blk = mode == 0 ? bi : 2;
  const BlockDesc d = a.desc[3 * ch.e + blk];
  const uint16_t *V = set ? d.Vs : d.V;
  const int R = set ? a.rs : a.r;
  const int K = d.K;
  const int i = 16 * it + (lane & 15);
  const int mloc = std::min(16 * sub + (lane & 15), ch.cnt - 1);
  const int pos = ch.base + mloc;
  const uint16_t *arow = (mode == 0) ? a.x + (int64_t)(a.sorted_pairs[pos] / a.k) * a.H
                                     : a.h + (int64_t)pos * a.I;
  arow += 8 * (lane >> 4);
  const uint16_t *vrow = V + (int64_t)std::min(i, R - 1) * K + 8 * (lane >> 4);
  const bool vi = i < R;
  const int nsteps = K / 32;
  const int s0 = nsteps * wave / 4, s1 = nsteps * (wave + 1) / 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int st = s0; st < s1; ++st) {
    f16x8 b = vi ? load_a(vrow + 32 * st) : pack_b(0, 0, 0, 0);
    acc = mfma16(load_a(arow + 32 * st), b, acc);
  }
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
  uint16_t *zbase = mode == 0 ? a.z_gu : a.z_d;
  const int zstride = mode == 0 ? 2 * a.RZ : a.RZ;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = 16 * sub + 4 * (lane >> 4) + q;
    if (m < ch.cnt) {
      const int p2 = ch.base + m;
      const bool comp = (a.sorted_pairs[p2] % a.k) < a.n_comp;
      const f16 v = comp ? (f16)sum[q] : (f16)0.0f;
      zbase[(int64_t)p2 * zstride + bi * a.RZ + set * a.Rp + 16 * it + (lane & 15)] =
          __builtin_bit_cast(uint16_t, v);
    }
  }
}

// y[t] = sum_j g[t][j] * sum_s ypart[s][pair_pos[t*k+j]]; one thread per
// (token, 4 columns).
template <bool F32>
__global__ void __launch_bounds__(256) combine_kernel(FfnArgs a, void *y) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_t = a.H / 4;
  if (id >= (int64_t)a.T * per_t) return;
  const int t = (int)(id / per_t), c = (int)(id % per_t) * 4;
  f32x4 out = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < a.k; ++j) {
    const float g = a.gates[(int64_t)t * a.k + j];
    const int pos = a.pair_pos[(int64_t)t * a.k + j];
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.splits; ++s) {
      const f32x4 p = *reinterpret_cast<const f32x4 *>(a.ypart + ((int64_t)s * a.P + pos) * a.H + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] += p[q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = __builtin_fmaf(g, v[q], out[q]);
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

static inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Ws {
  size_t z_gu, z_d, h, ypart, total;
};

static int pick_splits(const moeq_layer *L, int T, int k, const moeq_ffn_options *o) {
  if (o && o->split_k > 0) return o->split_k;
  const int P = T * k;
  const int n_g4 = (L->dims.I / kTileK + 3) / 4;
  // few tokens: split the long down-projection K for more waves in flight
  int s = P <= 256 ? 4 : 1;
  return std::max(1, std::min(s, n_g4));
}

static Ws ws_plan(const moeq_layer *L, int T, int k, int splits) {
  const int64_t P = (int64_t)T * k;
  const int Rp = (L->dims.r + 31) / 32 * 32, Rsp = (L->dims.rs + 31) / 32 * 32;
  const int RZ = Rp + Rsp;
  Ws w;
  size_t off = 0;
  w.z_gu = off; off = al256(off + (size_t)P * 2 * RZ * 2);
  w.z_d = off; off = al256(off + (size_t)P * RZ * 2);
  w.h = off; off = al256(off + (size_t)P * L->dims.I * 2);
  w.ypart = off; off = al256(off + (size_t)splits * P * L->dims.H * 4);
  w.total = off;
  return w;
}

static int max_chunks(int E, int T, int k) {
  const int64_t P = (int64_t)T * k;
  const int64_t a = (int64_t)E * ((T + kMT - 1) / kMT);
  const int64_t act = std::min<int64_t>(E, P);
  const int64_t b = (P + act * (kMT - 1)) / kMT;
  return (int)std::max<int64_t>(0, std::min(a, b));
}

}  // namespace moeq

using namespace moeq;

MOEQ_API moeq_status moeq_ffn_workspace_size(const moeq_layer *L, int32_t T, int32_t k,
                                             const moeq_ffn_options *opts, size_t *bytes) {
  if (!L || !bytes) return fail(MOEQ_ERR_INVALID, "ffn_workspace_size: null argument");
  if (T < 0 || k < 1 || k > L->dims.E) return fail(MOEQ_ERR_INVALID, "ffn_workspace_size: T=%d k=%d invalid", T, k);
  if (opts && (opts->split_k < 0 || opts->split_k > 64)) return fail(MOEQ_ERR_INVALID, "ffn_workspace_size: split_k=%d not in 0..64", opts->split_k);
  *bytes = ws_plan(L, T, k, pick_splits(L, T, k, opts)).total;
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_expert_ffn(const moeq_layer *L, const uint16_t *x, int32_t T, int32_t k,
                                     const moeq_routing *r, int32_t n_comp, void *y, int32_t y_dtype,
                                     void *ws, size_t ws_bytes, const moeq_ffn_options *opts,
                                     hipStream_t stream) {
  if (!L || !r) return fail(MOEQ_ERR_INVALID, "expert_ffn: null layer or routing");
  const LayerDims &D = L->dims;
  if (T < 0 || k < 1 || k > D.E) return fail(MOEQ_ERR_INVALID, "expert_ffn: T=%d k=%d invalid for E=%d", T, k, D.E);
  if (n_comp < 0 || n_comp > k) return fail(MOEQ_ERR_INVALID, "expert_ffn: n_comp=%d not in 0..%d", n_comp, k);
  if (y_dtype != MOEQ_F16 && y_dtype != MOEQ_F32) return fail(MOEQ_ERR_INVALID, "expert_ffn: bad y_dtype %d", y_dtype);
  const int path = opts ? opts->path : MOEQ_PATH_AUTO;
  if (path != MOEQ_PATH_AUTO && path != MOEQ_PATH_STREAM)
    return fail(MOEQ_ERR_UNSUPPORTED, "expert_ffn: path %d not available", path);
  if (opts && (opts->split_k < 0 || opts->split_k > 64)) return fail(MOEQ_ERR_INVALID, "expert_ffn: split_k=%d not in 0..64", opts->split_k);
  if (T == 0) return MOEQ_OK;
  if (!x || !y || !r->topk_gates || !r->expert_offsets || !r->sorted_pairs || !r->pair_pos)
    return fail(MOEQ_ERR_INVALID, "expert_ffn: null pointer");
  const int splits = pick_splits(L, T, k, opts);
  const Ws w = ws_plan(L, T, k, splits);
  if (!ws || ws_bytes < w.total)
    return fail(MOEQ_ERR_WORKSPACE, "expert_ffn: workspace has %zu bytes, needs %zu", ws_bytes, w.total);

  uint8_t *wb = static_cast<uint8_t *>(ws);
  FfnArgs a;
  a.desc = L->d_desc;
  a.offsets = r->expert_offsets;
  a.sorted_pairs = r->sorted_pairs;
  a.x = x;
  a.gates = r->topk_gates;
  a.pair_pos = r->pair_pos;
  a.E = D.E; a.H = D.H; a.I = D.I; a.k = k; a.T = T; a.n_comp = n_comp;
  a.r = D.r; a.rs = D.rs;
  a.Rp = (D.r + 31) / 32 * 32; a.Rsp = (D.rs + 31) / 32 * 32; a.RZ = a.Rp + a.Rsp;
  a.comp_on = (n_comp > 0 && a.RZ > 0) ? 1 : 0;
  a.z_gu = reinterpret_cast<uint16_t *>(wb + w.z_gu);
  a.z_d = reinterpret_cast<uint16_t *>(wb + w.z_d);
  a.h = reinterpret_cast<uint16_t *>(wb + w.h);
  a.ypart = reinterpret_cast<float *>(wb + w.ypart);
  a.splits = splits;
  a.P = T * k;

  const int mc = max_chunks(D.E, T, k);
  const bool g64 = D.fmt == MOEQ_FMT_INT && D.G == 64;
  if (a.comp_on) {
    prof_begin("lowrank_project_gu", stream);
    hipLaunchKernelGGL(lowrank_project_kernel, dim3(mc * kSub, 2 * a.RZ / 16), dim3(256), 0, stream, a, 0);
    prof_end("lowrank_project_gu", stream);
  }
  prof_begin("gateup_stream", stream);
  if (g64) hipLaunchKernelGGL(gateup_stream_kernel<2>, dim3(mc * (D.I / 64)), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(gateup_stream_kernel<1>, dim3(mc * (D.I / 64)), dim3(256), 0, stream, a);
  prof_end("gateup_stream", stream);
  if (a.comp_on) {
    prof_begin("lowrank_project_down", stream);
    hipLaunchKernelGGL(lowrank_project_kernel, dim3(mc * kSub, a.RZ / 16), dim3(256), 0, stream, a, 1);
    prof_end("lowrank_project_down", stream);
  }
  prof_begin("down_stream", stream);
  if (g64) hipLaunchKernelGGL(down_stream_kernel<2>, dim3(mc * (D.H / 64) * splits), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(down_stream_kernel<1>, dim3(mc * (D.H / 64) * splits), dim3(256), 0, stream, a);
  prof_end("down_stream", stream);
  prof_begin("combine", stream);
  const int64_t nthreads = (int64_t)T * (D.H / 4);
  if (y_dtype == MOEQ_F32)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, stream, a, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, stream, a, y);
  prof_end("combine", stream);
  return check_launch("expert_ffn");
}
