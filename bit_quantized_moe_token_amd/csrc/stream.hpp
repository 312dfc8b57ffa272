// Weight-streaming expert GEMMs: gate/up (+ low-rank epilogue + SwiGLU) and
// down (+ low-rank epilogue, split-K).  PagedWeight review summary: one
// fused kernel executes the per-block variable bitwidths; MxMoE abstract:
// per-linear-block bitwidths and uneven tokens per expert; TileQ abstract:
// the low-rank terms fused into the expert pass.
//
// A workgroup = 4 waves = 4 strips of 16 output rows of one expert, for one
// chunk of up to 32 of the expert's tokens (NSUB 16-row MFMA tiles).  Every
// packed weight is read from HBM exactly once per chunk.  K is walked in
// groups of four 128-column tiles:
//   - the group's activations (NSUB*16 rows x 512 columns, rows gathered by
//     token) sit in LDS, row stride padded by 16 B so that the MFMA A reads
//     are bank-conflict free;
//   - each wave loads the group's packed codes (128-bit loads) and metadata
//     into registers, then the next group's activations (so that waiting
//     for the codes never waits for them); several resident workgroups per
//     SIMD cover the HBM latency;
//   - the group is decoded in registers and fed to v_mfma_f32_16x16x32_f16
//     (B = decoded weights, A = activations from LDS).  INT blocks produce
//     exact (c - z) operands and apply the fp16 scale to each quantization
//     group's fp32 sum; bit-plane blocks look their q-bit indices up in
//     per-row LUTs staged in LDS.
// Bitwidths are template parameters: the kernel entry dispatches on the
// (gate, up) or down bitwidths of the chunk's expert.
#pragma once
#include "common.hpp"
#include "decode.hpp"
#include "ffn.hpp"
#include "layer.hpp"

namespace moeq {

constexpr int kXStride = 4 * kTileK + 8;   // halves per staged activation row
constexpr int kH32Stream = 64 + 4;          // floats per row of the gate/up epilogue's fp32 h tile

// Staging buffers per class: the 16-token INT class (occupancy 4 by
// registers) has LDS to spare for two, which saves one barrier per tile
// group; the larger classes and the bit-plane kernels (per-wave LUTs in
// LDS) keep one.  Sizes of one buffer: activations (halves) and per-group
// column sums (floats, 4 tiles x up to 2 groups x rows).
template <int NSUB, bool PLANE>
__host__ __device__ constexpr int xs_bufs() { return NSUB == 1 && !PLANE ? 2 : 1; }
template <int NSUB>
__host__ __device__ constexpr int xs_halves() { return NSUB * 16 * kXStride; }
template <int NSUB>
__host__ __device__ constexpr int sx_floats() { return 8 * NSUB * 16; }
constexpr int kLutBlk = 4 * 16 * 16;       // halves of one block's staged LUTs (4 tiles x 16 rows x 16)

// Packed data of one strip of one block for one group of C tiles.
template <int B, bool PLANE>
struct Group {
  static constexpr int NW = PLANE ? 4 * B : 4 * B;   // INT: 4 tiles x B dwords; planes: B planes x 4 tiles
  uint32_t w[NW];
  uint32_t sc[4];   // INT: fp16 scale of (tile t, group gi) at half t*GPT+gi
  uint32_t zz[2];   // INT: zero of (tile t, group gi) at byte t*GPT+gi
};

template <int B, int C, int GPT>
__device__ __forceinline__ void load_int_meta(const BlockDesc &d, int strip, int g4, int n_kt, Group<B, false> &g) {
  const int r = threadIdx.x & 15;
  const uint64_t mi = meta_index(strip, 4 * g4, r, 0, n_kt, GPT);
  const uint16_t *sp = d.scales + mi;
  const uint8_t *zp = d.zeros + mi;
  if (C == 4 && GPT == 1) {
    const u32x2 v = gld<u32x2>(sp);
    g.sc[0] = v[0]; g.sc[1] = v[1];
    g.zz[0] = gld<uint32_t>(zp);
  } else if (C == 4 && GPT == 2) {
    const u32x4 v = gld<u32x4>(sp);
    g.sc[0] = v[0]; g.sc[1] = v[1]; g.sc[2] = v[2]; g.sc[3] = v[3];
    const u32x2 z = gld<u32x2>(zp);
    g.zz[0] = z[0]; g.zz[1] = z[1];
  } else {
    g.sc[0] = g.sc[1] = g.sc[2] = g.sc[3] = 0;
    g.zz[0] = g.zz[1] = 0;
#pragma unroll
    for (int q = 0; q < C * GPT; ++q) {
      g.sc[q >> 1] |= (uint32_t)gld<uint16_t>(sp + q) << (16 * (q & 1));
      g.zz[q >> 2] |= (uint32_t)gld<uint8_t>(zp + q) << (8 * (q & 3));
    }
  }
}

template <int B, int C, int GPT>
__device__ __forceinline__ void load_int_group(const BlockDesc &d, int strip, int g4, int n_kt, Group<B, false> &g) {
  const int lane = threadIdx.x & 63;
  const uint8_t *p = d.codes + int_word_offset(strip, 4 * g4, lane, 0, n_kt, B);
  if (C == 4) {
    // chunk i of the group: 1 KiB of consecutive bytes across the wave
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const u32x4 v = gld_nt<u32x4>(p + 1024 * i);
      g.w[4 * i] = v[0]; g.w[4 * i + 1] = v[1]; g.w[4 * i + 2] = v[2]; g.w[4 * i + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < C * B; ++i) g.w[i] = gld<uint32_t>(p + 4 * i);
  }
  load_int_meta<B, C, GPT>(d, strip, g4, n_kt, g);
}

template <int Q, int C>
__device__ __forceinline__ void load_plane_group(const BlockDesc &d, int strip, int g4, int n_kt, Group<Q, true> &g) {
  const int lane = threadIdx.x & 63;
  const uint64_t off = code_offset(strip, 4 * g4, lane, n_kt, 4);
#pragma unroll
  for (int u = 0; u < Q; ++u) {
    const uint8_t *p = d.codes + u * d.plane_bytes + off;
    if (C == 4) {
      const u32x4 v = gld<u32x4>(p);
      g.w[4 * u] = v[0]; g.w[4 * u + 1] = v[1]; g.w[4 * u + 2] = v[2]; g.w[4 * u + 3] = v[3];
    } else {
#pragma unroll
      for (int t = 0; t < C; ++t) g.w[4 * u + t] = gld<uint32_t>(p + 4 * t);
    }
  }
}

template <int B, bool PLANE, int C, int GPT>
__device__ __forceinline__ void load_group(const BlockDesc &d, int strip, int g4, int n_kt, Group<B, PLANE> &g) {
  if constexpr (PLANE) load_plane_group<B, C>(d, strip, g4, n_kt, g);
  else load_int_group<B, C, GPT>(d, strip, g4, n_kt, g);
}

// A operand of token tile s, tile tl, step j from the staged activations.
__device__ __forceinline__ f16x8 lds_a(const uint16_t *xs, int s, int tl, int j) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const f16x8 *>(xs + (16 * s + (lane & 15)) * kXStride + tl * kTileK +
                                          32 * j + 8 * (lane >> 4));
}

__device__ __forceinline__ uint32_t int_zero(const uint32_t *zz, int q) {
  return (zz[q >> 2] >> (8 * (q & 3))) & 0xffu;
}
__device__ __forceinline__ float int_scale(const uint32_t *sc, int q) {
  return (float)__builtin_bit_cast(f16, (uint16_t)(sc[q >> 1] >> (16 * (q & 1))));
}

// One group of C tiles for NB INT blocks sharing the A operands: each
// activation fragment read from LDS feeds the MFMAs of every block before
// the next is read.  The staged activations are pre-scaled for b0's field
// pattern (block 1 re-scales a fragment to its own pattern when its
// bitwidth differs), so the subnormal-form B operands give, per
// quantization group and token subtile, P_b = 2^-24 sum c x.  With
// S = -2^-24 sum x of the group's columns (per token, staged in LDS next to
// the activations), acc_b += s_b (P_b + z_b S) = 2^-24 s_b sum (c - z) x.
// The accumulators stay in units of 2^-24 until the end of the K walk.
template <int NSUB, int NB, int B0, int B1, int C, int GPT>
__device__ __forceinline__ void compute_int(const Group<B0, false> &g0, const Group<B1, false> &g1,
                                            const uint16_t *xs, const float *sx, f32x4 (*acc)[NSUB]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int tl = 0; tl < C; ++tl) {
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      const int q = tl * GPT + gi;
      f32x4 p0[NSUB], p1[NSUB];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) { p0[s] = f32x4{0.f, 0.f, 0.f, 0.f}; p1[s] = p0[s]; }
#pragma unroll
      for (int jj = 0; jj < 4 / GPT; ++jj) {
        const int j = gi * (4 / GPT) + jj;
        const f16x8 b0 = int_bop_sub<B0>(g0.w + tl * B0, j);
        f16x8 b1;
        if (NB == 2) b1 = int_bop_sub<B1>(g1.w + tl * B1, j);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          const f16x8 av = lds_a(xs, s, tl, j);
          p0[s] = mfma16(av, b0, p0[s]);
          if (NB == 2) p1[s] = mfma16(rescale_a<B0, B1>(av), b1, p1[s]);
        }
      }
      const float z0 = (float)int_zero(g0.zz, q), s0 = int_scale(g0.sc, q);
      const float z1 = NB == 2 ? (float)int_zero(g1.zz, q) : 0.f;
      const float s1 = NB == 2 ? int_scale(g1.sc, q) : 0.f;
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const f32x4 sv = *reinterpret_cast<const f32x4 *>(sx + q * (NSUB * 16) + 16 * s + 4 * (lane >> 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[0][s][i] = __builtin_fmaf(s0, __builtin_fmaf(z0, sv[i], p0[s][i]), acc[0][s][i]);
          if (NB == 2) acc[1][s][i] = __builtin_fmaf(s1, __builtin_fmaf(z1, sv[i], p1[s][i]), acc[1][s][i]);
        }
        // keep the group's update here (not sunk past later groups), so its
        // partial sums die at once
        asm volatile("" : "+v"(acc[0][s]), "+v"(acc[1][s]));
      }
    }
  }
}

// Decoded B operand of step j from the top q planes and the lane's row LUT
// (byte-split: low bytes of the entries, then high bytes): two quads of
// four weights, each looked up by byte permutes.
template <int Q>
__device__ __forceinline__ f16x8 plane_bop(const uint32_t *tp, int j, const uint32_t *L) {
  uint32_t d[4];
  plane_quad<Q>(tp, j, L, d[0], d[1]);
  plane_quad<Q>(tp, 4 + j, L, d[2], d[3]);
  return pack_b(d[0], d[1], d[2], d[3]);
}

template <int Q>
__device__ __forceinline__ void lut_row(const uint16_t *lut, int tl, uint32_t *L) {
  constexpr int NQ = 1 << Q;
  const int lane = threadIdx.x & 63;
  const uint32_t *lp = reinterpret_cast<const uint32_t *>(lut + (tl * 16 + (lane & 15)) * NQ);
#pragma unroll
  for (int i = 0; i < NQ / 2; ++i) L[i] = lp[i];
}

template <int NSUB, int NB, int Q0, int Q1, int C>
__device__ __forceinline__ void compute_plane(const Group<Q0, true> &g0, const Group<Q1, true> &g1,
                                              const uint16_t *xs, const uint16_t *lut, f32x4 (*acc)[NSUB]) {
#pragma unroll
  for (int tl = 0; tl < C; ++tl) {
    uint32_t L0[1 << (Q0 - 1)], L1[1 << (Q1 - 1)];
    lut_row<Q0>(lut, tl, L0);
    if (NB == 2) lut_row<Q1>(lut + kLutBlk, tl, L1);
    uint32_t t0[Q0], t1[Q1];
#pragma unroll
    for (int u = 0; u < Q0; ++u) t0[u] = g0.w[4 * u + tl];
#pragma unroll
    for (int u = 0; u < Q1; ++u) t1[u] = NB == 2 ? g1.w[4 * u + tl] : 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x8 b0 = plane_bop<Q0>(t0, j, L0);
      f16x8 b1;
      if (NB == 2) b1 = plane_bop<Q1>(t1, j, L1);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const f16x8 av = lds_a(xs, s, tl, j);
        acc[0][s] = mfma16(av, b0, acc[0][s]);
        if (NB == 2) acc[1][s] = mfma16(av, b1, acc[1][s]);
      }
    }
  }
}

// ---- activation staging: NSUB*16 rows x 512 columns of group g4, by all
// NW waves of the workgroup.  Pass p loads row NW*p + wave (wave-uniform
// row pointer); a lane moves 16 B.
template <int NSUB, int NW>
struct XStage {
  static constexpr int NP = NSUB * 16 / NW;
  u32x4 v[NP];
};

// Lanes past the group's c tiles (ragged last group) re-read the group's
// first columns instead of branching; their LDS columns are never read.
template <int NSUB, int NW>
__device__ __forceinline__ void stage_load(XStage<NSUB, NW> &st, const uint16_t *const *rowp, int g4, int c) {
  const int lane = threadIdx.x & 63;
  const int col = 4 * kTileK * g4 + 8 * (lane < 16 * c ? lane : 0);      // halves
#pragma unroll
  for (int p = 0; p < XStage<NSUB, NW>::NP; ++p) st.v[p] = gld<u32x4>(rowp[p] + col);
}

// One DPP lane permutation of a float (ctrl: a DPP control constant).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

// Sum of a float over the lanes of each DPP row (16 lanes) or half-row (8).
template <int LANES>
__device__ __forceinline__ float row_sum(float t) {
  t += dpp_f<0xb1>(t);                         // quad_perm [1,0,3,2]
  t += dpp_f<0x4e>(t);                         // quad_perm [2,3,0,1]
  t += dpp_f<0x141>(t);                        // row_half_mirror
  if constexpr (LANES == 16) t += dpp_f<0x140>(t);   // row_mirror
  return t;
}

// PS > 0 (INT codes of PS bits): besides storing the row, write
// S = -2^-24 * (sum of the row's columns) per quantization group (GPT per
// tile) to sx[(tile * GPT + group) * NSUB*16 + row], then pre-scale the
// columns for the field pattern (dword v of a lane's 16 bytes holds the two
// columns of register v).  Lane l holds columns 8l..8l+7 of the 4-tile row,
// so the 16 lanes of a DPP row are one tile.  The staged rows are
// normalised (x~ = x 2^K, or h~; largest magnitude in [2^6, 2^7)), so the
// pre-scale makes a value subnormal only below 2^-21 of its row's largest.
template <int NSUB, int NW, int PS, int GPT>
__device__ __forceinline__ void stage_store(const XStage<NSUB, NW> &st, uint16_t *xs, float *sx, int c) {
  (void)c;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int p = 0; p < XStage<NSUB, NW>::NP; ++p) {
    const int row = NW * p + wave;
    u32x4 v = st.v[p];
    if constexpr (PS > 0) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) t = __builtin_amdgcn_fdot2(as_h2(v[w]), f16x2{1.0f16, 1.0f16}, t, false);
      constexpr int L = 16 / GPT;
      t = row_sum<L>(t);
      if ((lane & (L - 1)) == 0) sx[(lane / L) * (NSUB * 16) + row] = t * -0x1p-24f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v[w] = prescale_pair<PS>(v[w], w);
    }
    *reinterpret_cast<u32x4 *>(xs + row * kXStride + 8 * lane) = v;
  }
}

// LUT staging of one wave's strip for a group: 4 tiles x 16 rows x NQ
// halves, contiguous in the packed LUT; lane l holds 2*NQ bytes.
template <int Q>
struct LutStage {
  uint32_t v[1 << (Q - 1)];
};

template <int Q>
__device__ __forceinline__ void lut_load(const BlockDesc &d, int strip, int g4, int n_kt, int c, LutStage<Q> &ls) {
  constexpr int NQ = 1 << Q;
  const int lane = threadIdx.x & 63;
  const uint16_t *p = d.lut + lut_index(strip, 4 * g4, 0, 0, n_kt, NQ) + (lane < 16 * c ? lane : 0) * NQ;
#pragma unroll
  for (int i = 0; i < NQ / 2; ++i) ls.v[i] = gld<uint32_t>(p + 2 * i);
}

// Stored byte-split for the permute lookups: the row's 2^q low bytes
// (entry i in byte i) in 2^q / 4 dwords, then its 2^q high bytes.
template <int Q>
__device__ __forceinline__ void lut_store(const LutStage<Q> &ls, uint16_t *dst, int c) {
  (void)c;
  constexpr int NQ = 1 << Q;
  const int lane = threadIdx.x & 63;
  uint32_t *row = reinterpret_cast<uint32_t *>(dst + lane * NQ);
#pragma unroll
  for (int m = 0; m < NQ / 4; ++m) {
    row[m] = __builtin_amdgcn_perm(ls.v[2 * m + 1], ls.v[2 * m], 0x06040200u);
    row[NQ / 4 + m] = __builtin_amdgcn_perm(ls.v[2 * m + 1], ls.v[2 * m], 0x07050301u);
  }
}

// Sum of the KS fp32 partials of four z columns (all loads issued before
// the first add).
__device__ __forceinline__ f32x4 zsum(const float *src, int64_t kstride, int KS) {
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 4 <= KS; k += 4) {
    const f32x4 v0 = gld<f32x4>(src + (k + 0) * kstride), v1 = gld<f32x4>(src + (k + 1) * kstride);
    const f32x4 v2 = gld<f32x4>(src + (k + 2) * kstride), v3 = gld<f32x4>(src + (k + 3) * kstride);
#pragma unroll
    for (int i = 0; i < 4; ++i) sum[i] += v0[i] + v1[i] + v2[i] + v3[i];
  }
  for (; k < KS; ++k) {
    const f32x4 v = gld<f32x4>(src + k * kstride);
#pragma unroll
    for (int i = 0; i < 4; ++i) sum[i] += v[i];
  }
  return sum;
}

// z of the chunk's pairs in LDS, rounded to fp16: the sum of the ks fp32
// partials of the projection kernel; zero for a pair outside its token's
// leading n_comp slots and in the rank padding.
//   gate/up (xk): scaled by 2^K of the row's token (z of the normalised
//   x~ = x 2^K); rows by sorted position, or (z_tok) by (token, expert)
//   (the group's leader has written the shared part into every member's
//   row).
//   down: the shared part is w' for the down leader of (token, group) —
//   the sum of its members' sub-rows — and 0 for the other pairs.
// zs layout: [NSUB*16 rows][width] fp16 with width = nset * RZ (RZ padded
// columns per block, the per-expert Rp first, then the shared Rsp).
template <int NSUB, int NW>
__device__ __forceinline__ void z_prologue(const FfnArgs &a, bool xk, const float *zpart, int zstride,
                                           int64_t kstride, int KS, int width, const Chunk &ch, uint16_t *zs) {
  const int tid = threadIdx.x;
  const int n4 = NSUB * 16 * width / 4;                  // float4 outputs
  for (int o = tid; o < n4; o += NW * 64) {
    const int row = (4 * o) / width, col = (4 * o) % width;
    const int m = std::min(row, ch.cnt - 1);
    const int pr = a.sorted_pairs[ch.base + m];
    const int t = pr / a.k;
    const bool shared = col % a.RZ >= a.Rp;
    // rank padding (ranks are multiples of 8, so a float4 is padding or
    // not as a whole) is zero and never read
    const bool pad = shared ? col % a.RZ - a.Rp >= a.rs : col % a.RZ >= a.r;
    const bool live = pr % a.k < a.n_comp && !pad;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    if (live) {
      if (shared && !xk) {
        // the leader's own sub-row (read with its member mask, in one round
        // trip), then the other members' (a group of several members is
        // the rarer case)
        const int pos = ch.base + m, js = pr % a.k;
        const float *src = a.zsh + (int64_t)pos * a.k * a.Rsp + (col - a.Rp);
        const uint32_t mask = (uint32_t)a.dlead[pos];
        const f32x4 own = zsum(src + js * a.Rsp, a.ks_stride_sh, KS);
        if (mask) {
          sum = own;
          for (uint32_t rest = mask & ~(1u << js); rest; rest &= rest - 1) {
            const f32x4 v = zsum(src + __builtin_ctz(rest) * a.Rsp, a.ks_stride_sh, KS);
#pragma unroll
            for (int i = 0; i < 4; ++i) sum[i] += v[i];
          }
        }
      } else {
        const int64_t srow = (xk && a.z_tok) ? (int64_t)t * a.E + ch.e : (int64_t)(ch.base + m);
        sum = zsum(zpart + srow * zstride + col, kstride, KS);
        if (xk) {
          const int K = a.xexp[t];
#pragma unroll
          for (int i = 0; i < 4; ++i) sum[i] = __builtin_ldexpf(sum[i], K);
        }
      }
    }
    u32x2 h;
    h[0] = as_u32(f16x2{(f16)sum[0], (f16)sum[1]});
    h[1] = as_u32(f16x2{(f16)sum[2], (f16)sum[3]});
    *reinterpret_cast<u32x2 *>(zs + row * width + col) = h;
  }
}

// B operand of U for z columns 32 ks .. 32 ks + 31 of output row `row`
// (zero past the rank R).
__device__ __forceinline__ f16x8 lowrank_bop(const uint16_t *U, int R, int row, int ks) {
  const int col = 32 * ks + 8 * ((threadIdx.x & 63) >> 4);
  return col < R ? load_a(U + (int64_t)row * R + col) : pack_b(0, 0, 0, 0);
}

// z rows of a chunk held in registers from before the K walk until the
// epilogue (one fp32 partial, width <= 8 * NW * 64 * 4 / (NSUB * 16)): the
// same values z_prologue would load, without its wait at the end.
template <int NSUB, int NW, int NV>
struct ZPre {
  f32x4 v[NV];
};

template <int NSUB, int NW, int NV>
__device__ __forceinline__ void z_preload(const float *zpart, int zstride, int width, const Chunk &ch,
                                          ZPre<NSUB, NW, NV> &zp) {
  const int tid = threadIdx.x;
  const int n4 = NSUB * 16 * width / 4;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int o = tid + i * NW * 64;
    const int row = (4 * o) / width, col = (4 * o) % width;
    const int m = std::min(row, ch.cnt - 1);
    zp.v[i] = o < n4 ? gld<f32x4>(zpart + (int64_t)(ch.base + m) * zstride + col) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// z_store scales row r by 2^kx[r] (kx: the rows' x exponents in LDS).
template <int NSUB, int NW, int NV>
__device__ __forceinline__ void z_store(const FfnArgs &a, const Chunk &ch, const int *kx, const ZPre<NSUB, NW, NV> &zp,
                                       int width, uint16_t *zs) {
  (void)a;
  (void)ch;
  const int tid = threadIdx.x;
  const int n4 = NSUB * 16 * width / 4;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int o = tid + i * NW * 64;
    if (o < n4) {
      const int row = (4 * o) / width, col = (4 * o) % width;
      const int K = kx[row];
      u32x2 h;
      h[0] = as_u32(f16x2{(f16)__builtin_ldexpf(zp.v[i][0], K), (f16)__builtin_ldexpf(zp.v[i][1], K)});
      h[1] = as_u32(f16x2{(f16)__builtin_ldexpf(zp.v[i][2], K), (f16)__builtin_ldexpf(zp.v[i][3], K)});
      *reinterpret_cast<u32x2 *>(zs + row * width + col) = h;
    }
  }
}

// Low-rank epilogue: acc += U z for one factor set (z rows in LDS, zero for
// uncompensated pairs and for columns >= R).  b0: the operand of the first
// 32 columns, loaded by the caller (the streaming kernels load it before
// their K walk, so the epilogue does not wait for it).
template <int NSUB>
__device__ __forceinline__ void lowrank_epi(const uint16_t *U, int R, int Rpad, int row, const uint16_t *zs,
                                            int zwidth, f32x4 *acc, f16x8 b0) {
  const int lane = threadIdx.x & 63, kq = lane >> 4;
  for (int ks = 0; ks < Rpad / 32; ++ks) {
    const int col = 32 * ks + 8 * kq;
    const f16x8 bop = ks == 0 ? b0 : lowrank_bop(U, R, row, ks);
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
      acc[s] = mfma16(*reinterpret_cast<const f16x8 *>(zs + (16 * s + (lane & 15)) * zwidth + col), bop, acc[s]);
  }
}

template <int NSUB>
__device__ __forceinline__ void lowrank_epi(const uint16_t *U, int R, int Rpad, int row, const uint16_t *zs,
                                            int zwidth, f32x4 *acc) {
  lowrank_epi<NSUB>(U, R, Rpad, row, zs, zwidth, acc, lowrank_bop(U, R, row, 0));
}

// Stage group g's activations (and the two streams' bit-plane LUTs) into
// LDS: load, then (after the caller's barrier) store.
template <int NSUB, int NW, bool PLANE, int B0, int B1, int GPT>
struct Stager {
  XStage<NSUB, NW> st;
  LutStage<B0> l0;
  LutStage<B1> l1;
  __device__ __forceinline__ void load(const BlockDesc &d0, const BlockDesc &d1, const uint16_t *const *rowp,
                                       int s0, int s1, int g4, int n_kt, int c) {
    stage_load<NSUB, NW>(st, rowp, g4, c);
    if constexpr (PLANE) {
      lut_load<B0>(d0, s0, g4, n_kt, c, l0);
      lut_load<B1>(d1, s1, g4, n_kt, c, l1);
    }
  }
  __device__ __forceinline__ void store(uint16_t *xs, float *sx, uint16_t *lut_lds, int c) {
    stage_store<NSUB, NW, PLANE ? 0 : B0, GPT>(st, xs, sx, c);
    if constexpr (PLANE) {
      lut_store<B0>(l0, lut_lds, c);
      lut_store<B1>(l1, lut_lds + kLutBlk, c);
    }
  }
};

template <int NSUB, int B0, int B1, bool PLANE, int C, int GPT>
__device__ __forceinline__ void compute_two(const Group<B0, PLANE> &g0, const Group<B1, PLANE> &g1,
                                            const uint16_t *xs, const float *sx, const uint16_t *lut,
                                            f32x4 (*acc)[NSUB]) {
  if constexpr (PLANE) compute_plane<NSUB, 2, B0, B1, C>(g0, g1, xs, lut, acc);
  else compute_int<NSUB, 2, B0, B1, C, GPT>(g0, g1, xs, sx, acc);
}

// Streams tile groups [g_begin, g_end) of two weight streams per wave —
// (block d0, strip s0) and (block d1, strip s1) — that share one activation
// fragment per MFMA.  The NW waves of the workgroup share the staged
// activations (and, for INT codes, the per-group column sums in sx).  Per
// group: this group's code loads first, then the next group's activations
// (publishing those never waits for the codes), then decode + MFMA; the
// other resident workgroups cover the load latency.  The codes of the
// first group (m0, m1, when it is a full group) are loaded by the caller
// before its prologue, so they arrive during it.
template <int NSUB, int NW, int GPT, bool PLANE, int B0, int B1>
__device__ __forceinline__ void stream_two(const BlockDesc &d0, const BlockDesc &d1, int s0, int s1,
                                           int g_begin, int g_end, const uint16_t *const *rowp, uint16_t *xs,
                                           float *sx, uint16_t *lut_lds, f32x4 (*acc)[NSUB],
                                           const Group<B0, PLANE> &m0, const Group<B1, PLANE> &m1) {
  const int n_kt = d0.K / kTileK;
  const int full = n_kt / 4;                   // groups with 4 tiles
  const int g_full_end = std::min(g_end, full);
  // staging buffers of group g (two alternate when the LDS allows: then
  // one barrier per group suffices, see group_step)
  constexpr int NXB = xs_bufs<NSUB, PLANE>();
  auto xb = [&](int g) { return xs + (NXB == 2 ? (g & 1) * xs_halves<NSUB>() : 0); };
  auto sb = [&](int g) { return sx + (NXB == 2 ? (g & 1) * sx_floats<NSUB>() : 0); };
  Stager<NSUB, NW, PLANE, B0, B1, GPT> stg;
  {
    const int c = std::min(4, n_kt - 4 * g_begin);
    stg.load(d0, d1, rowp, s0, s1, g_begin, n_kt, c);
    stg.store(xb(g_begin), sb(g_begin), lut_lds, c);
    __syncthreads();
  }
  // one full group: the next group's activations load, this group is
  // decoded and multiplied, then the activations are published.  With one
  // buffer the store waits for every wave to finish reading it; with two it
  // goes to the buffer that the barrier of the previous group already
  // freed, and the one barrier after it publishes it.  (Bit-plane LUTs are
  // per wave: a wave overwrites only rows it has finished reading.)
  auto group_step = [&](int g, const Group<B0, PLANE> &c0, const Group<B1, PLANE> &c1) {
    const bool more = g + 1 < g_end;
    const int cn = more ? std::min(4, n_kt - 4 * (g + 1)) : 0;
    if (more) stg.load(d0, d1, rowp, s0, s1, g + 1, n_kt, cn);
    compute_two<NSUB, B0, B1, PLANE, 4, GPT>(c0, c1, xb(g), sb(g), lut_lds, acc);
    if (more) {
      if constexpr (NXB == 1) __syncthreads();
      stg.store(xb(g + 1), sb(g + 1), lut_lds, cn);
      __syncthreads();
    }
  };
  if (g_begin < g_full_end) {
    group_step(g_begin, m0, m1);               // codes loaded by the caller up front
#pragma unroll 1
    for (int g = g_begin + 1; g < g_full_end; ++g) {
      Group<B0, PLANE> c0;
      Group<B1, PLANE> c1;
      load_group<B0, PLANE, 4, GPT>(d0, s0, g, n_kt, c0);
      load_group<B1, PLANE, 4, GPT>(d1, s1, g, n_kt, c1);
      group_step(g, c0, c1);
    }
  }
  if (g_end > full) {                          // the ragged last group
    Group<B0, PLANE> t0;
    Group<B1, PLANE> t1;
    switch (n_kt - 4 * full) {
      case 1:
        load_group<B0, PLANE, 1, GPT>(d0, s0, full, n_kt, t0); load_group<B1, PLANE, 1, GPT>(d1, s1, full, n_kt, t1);
        compute_two<NSUB, B0, B1, PLANE, 1, GPT>(t0, t1, xb(full), sb(full), lut_lds, acc); break;
      case 2:
        load_group<B0, PLANE, 2, GPT>(d0, s0, full, n_kt, t0); load_group<B1, PLANE, 2, GPT>(d1, s1, full, n_kt, t1);
        compute_two<NSUB, B0, B1, PLANE, 2, GPT>(t0, t1, xb(full), sb(full), lut_lds, acc); break;
      default:
        load_group<B0, PLANE, 3, GPT>(d0, s0, full, n_kt, t0); load_group<B1, PLANE, 3, GPT>(d1, s1, full, n_kt, t1);
        compute_two<NSUB, B0, B1, PLANE, 3, GPT>(t0, t1, xb(full), sb(full), lut_lds, acc); break;
    }
  }
  if constexpr (!PLANE) {                      // INT sums are in units of 2^-24
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[b][s] *= 16777216.0f;
  }
}

// Codes of group g of two streams, loaded up front when g is a full group.
template <int GPT, bool PLANE, int B0, int B1>
__device__ __forceinline__ void preload_two(const BlockDesc &d0, const BlockDesc &d1, int s0, int s1, int g,
                                            Group<B0, PLANE> &p0, Group<B1, PLANE> &p1) {
  const int n_kt = d0.K / kTileK;
  if (g < n_kt / 4) {
    load_group<B0, PLANE, 4, GPT>(d0, s0, g, n_kt, p0);
    load_group<B1, PLANE, 4, GPT>(d1, s1, g, n_kt, p1);
  }
}

// Wave-uniform row pointers of the staged activations: pass p loads chunk
// row NW*p + wave (clamped to the last valid row): the token's normalised
// x~ row (gate/up) or the pair's normalised h row (down).
template <int NSUB, int NW>
__device__ __forceinline__ void row_ptrs(const uint16_t **rowp, const FfnArgs &a, const Chunk &ch, bool gather) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int p = 0; p < XStage<NSUB, NW>::NP; ++p) {
    const int m = std::min(NW * p + wave, ch.cnt - 1);
    const uint16_t *ptr;
    if (gather) ptr = a.xn + (int64_t)(a.sorted_pairs[ch.base + m] / a.k) * a.H;
    else ptr = a.hn + (int64_t)(ch.base + m) * a.I;
    const uint64_t u = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    rowp[p] = reinterpret_cast<const uint16_t *>(((uint64_t)hi << 32) | lo);
  }
}

// LDS layout of both stream kernels: [x staging | z rows (2 RZ columns) |
// per-group column sums (4 tiles x 2 groups x NSUB*16 rows, fp32) | per wave:
// its two streams' bit-plane LUTs (bit-plane kernels only)].  The gate/up
// epilogue reuses the staging area for its fp32 h tile.  The bit-plane
// kernels build their z rows after the K walk, in the staging area: their
// LUTs already hold them near the LDS limit, and the 8 KiB this saves make
// room for a third workgroup per CU.
template <bool PLANE>
__host__ __device__ constexpr bool z_late() { return PLANE; }
static_assert(2 * (64 + 64) <= kXStride, "z rows of the largest ranks fit a staged activation row");

template <int NSUB, bool PLANE>
__device__ __forceinline__ int zs_offset() { return z_late<PLANE>() ? 0 : xs_bufs<NSUB, PLANE>() * xs_halves<NSUB>(); }

template <int NSUB, bool PLANE>
__device__ __forceinline__ float *sx_region(uint16_t *lds, int RZ) {
  return reinterpret_cast<float *>(lds + xs_bufs<NSUB, PLANE>() * xs_halves<NSUB>() +
                                   (z_late<PLANE>() ? 0 : NSUB * 16 * 2 * RZ));
}

template <int NSUB, bool PLANE>
__device__ __forceinline__ uint16_t *lut_region(uint16_t *lds, int RZ, int wave) {
  return reinterpret_cast<uint16_t *>(sx_region<NSUB, PLANE>(lds, RZ) +
                                     xs_bufs<NSUB, PLANE>() * sx_floats<NSUB>()) + wave * 2 * kLutBlk;
}


// gate/up: 4 waves, each streams the gate and the up rows of one 16-row
// strip; h = SiLU(gate) * up is formed in registers.  The kernels work on
// the normalised x~ = x 2^K (one K per token), so the accumulators and the
// z rows (V x~) share its units; the epilogue returns to x's in fp32.  h is
// stored as fp16 h 2^(kNormTop - eb) with eb the exponent of the pair's
// largest |h| over the workgroup's 64 rows (block sg of I), and eb (int8)
// goes to hblk.
template <int NSUB, int GPT, bool PLANE, int BG, int BU>
__device__ __forceinline__ void gateup_body(const FfnArgs &a, const Chunk &ch, int strip, uint16_t *lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint16_t *xs = lds;
  uint16_t *zs = lds + zs_offset<NSUB, PLANE>();
  const int zw = 2 * a.RZ;
  const BlockDesc dg = a.desc[3 * ch.e], du = a.desc[3 * ch.e + 1];   // scalar loads
  Group<BG, PLANE> p0;
  Group<BU, PLANE> p1;
  preload_two<GPT, PLANE, BG, BU>(dg, du, strip, strip, 0, p0, p1);
  // the rows' pair ids and x exponents: requested now, kept in two
  // registers and put in LDS after the K walk (the epilogue reads them
  // there)
  const int preg = threadIdx.x < NSUB * 16 ? a.sorted_pairs[ch.base + std::min((int)threadIdx.x, ch.cnt - 1)] : 0;
  const int kreg = threadIdx.x < NSUB * 16 ? a.xexp[preg / a.k] : 0;
  if (!z_late<PLANE>() && a.comp_on) {
    z_prologue<NSUB, 4>(a, true, a.zp_gu, 2 * a.RZ, a.ks_stride_gu, a.ks_gu, zw, ch, zs);
    __syncthreads();
  }
  const uint16_t *rowp[XStage<NSUB, 4>::NP];
  row_ptrs<NSUB, 4>(rowp, a, ch, true);
  const int row = strip * 16 + (lane & 15);
  // first U operands (gate, up), requested before the K walk
  f16x8 ub[2] = {pack_b(0, 0, 0, 0), pack_b(0, 0, 0, 0)};
  if (a.comp_on && a.r > 0) {
    ub[0] = lowrank_bop(dg.U, a.r, row, 0);
    ub[1] = lowrank_bop(du.U, a.r, row, 0);
  }
  f32x4 acc[2][NSUB];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[b][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int n_g4 = (a.H / kTileK + 3) / 4;
  stream_two<NSUB, 4, GPT, PLANE, BG, BU>(dg, du, strip, strip, 0, n_g4, rowp, xs, sx_region<NSUB, PLANE>(lds, a.RZ),
                                          lut_region<NSUB, PLANE>(lds, a.RZ, wave), acc, p0, p1);
  // (the column sums' LDS is free once every wave has passed the barrier
  // below; the exponents go there)
  int *s_kx = reinterpret_cast<int *>(sx_region<NSUB, PLANE>(lds, a.RZ));
  int *s_p = s_kx + NSUB * 16;
  if (z_late<PLANE>() && a.comp_on) {
    __syncthreads();     // every wave is done with the staging area
    z_prologue<NSUB, 4>(a, true, a.zp_gu, 2 * a.RZ, a.ks_stride_gu, a.ks_gu, zw, ch, zs);
    __syncthreads();
  }
  if (a.comp_on) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const BlockDesc &d = b ? du : dg;
      if (a.r > 0) lowrank_epi<NSUB>(d.U, a.r, a.Rp, row, zs + b * a.RZ, zw, acc[b], ub[b]);
      if (a.rs > 0) lowrank_epi<NSUB>(d.Us, a.rs, a.Rsp, row, zs + b * a.RZ + a.Rp, zw, acc[b]);
    }
  }
  // h = SiLU(gate) * up (back in x's units) in fp32 into LDS [rows][64
  // columns] (the staging buffers are free once every wave has finished
  // its K walk), then coalesced: 8 threads (a DPP half-row) per token row
  // take its largest |h| over the workgroup's 64 columns for eb, and store
  // h 2^(kNormTop - eb) as fp16
  float *h32 = reinterpret_cast<float *>(lds);
  __syncthreads();
  if (threadIdx.x < NSUB * 16) {
    s_kx[threadIdx.x] = kreg;
    s_p[threadIdx.x] = preg;
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * s + 4 * (lane >> 4) + i;
      const int K = -s_kx[m];
      const float g = __builtin_ldexpf(acc[0][s][i], K), u = __builtin_ldexpf(acc[1][s][i], K);
      h32[m * kH32Stream + 16 * wave + (lane & 15)] = g / (1.0f + __expf(-g)) * u;
    }
  }
  __syncthreads();
  const int tid = threadIdx.x, sg = strip >> 2;
  if (tid < NSUB * 16 * 8) {
    const int m = tid >> 3, c8 = 8 * (tid & 7);
    const f32x4 v0 = *reinterpret_cast<const f32x4 *>(h32 + m * kH32Stream + c8);
    const f32x4 v1 = *reinterpret_cast<const f32x4 *>(h32 + m * kH32Stream + c8 + 4);
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fabsf(v0[j]), __builtin_fabsf(v1[j])));
    const int eb = h_block_exp(dpp_half_row_max(mx));
    if (m < ch.cnt) {
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        o[j] = as_u32(f16x2{(f16)__builtin_ldexpf(v0[2 * j], kNormTop - eb), (f16)__builtin_ldexpf(v0[2 * j + 1], kNormTop - eb)});
        o[2 + j] = as_u32(f16x2{(f16)__builtin_ldexpf(v1[2 * j], kNormTop - eb), (f16)__builtin_ldexpf(v1[2 * j + 1], kNormTop - eb)});
      }
      *reinterpret_cast<u32x4 *>(a.h + (int64_t)(ch.base + m) * a.I + 64 * sg + c8) = o;
      if ((tid & 7) == 0) {
        a.hblk[(int64_t)(ch.base + m) * a.hblk_stride + sg] = (int8_t)eb;
        h_pair_exp(a, ch.base + m, s_p[m], eb);
      }
    }
  }
}

// down: 4 waves, each streams two 16-row strips of the down block over the
// split's K range.
template <int NSUB, int GPT, bool PLANE, int BD>
__device__ __forceinline__ void down_body(const FfnArgs &a, const Chunk &ch, int sg, int split, uint16_t *lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint16_t *xs = lds;
  uint16_t *zs = lds + zs_offset<NSUB, PLANE>();
  const int zw = a.RZ;
  const bool epi = a.comp_on && split == 0;
  const BlockDesc d = a.desc[3 * ch.e + 2];                          // scalar loads
  const int n_g4 = (a.I / kTileK + 3) / 4;
  const int g0 = (int)((int64_t)n_g4 * split / a.splits);
  const int g1 = (int)((int64_t)n_g4 * (split + 1) / a.splits);
  const int st0 = 8 * sg + 2 * wave, st1 = st0 + 1;
  Group<BD, PLANE> p0, p1;
  if (g1 > g0) preload_two<GPT, PLANE, BD, BD>(d, d, st0, st1, g0, p0, p1);
  if (!z_late<PLANE>() && epi) {
    z_prologue<NSUB, 4>(a, false, a.zp_d, a.RZ, a.ks_stride_d, a.ks_d, zw, ch, zs);
    __syncthreads();
  }
  const uint16_t *rowp[XStage<NSUB, 4>::NP];
  row_ptrs<NSUB, 4>(rowp, a, ch, false);
  // first U operands of the two strips, requested before the K walk
  f16x8 ub[2] = {pack_b(0, 0, 0, 0), pack_b(0, 0, 0, 0)};
  if (epi && a.r > 0) {
    ub[0] = lowrank_bop(d.U, a.r, st0 * 16 + (lane & 15), 0);
    ub[1] = lowrank_bop(d.U, a.r, st1 * 16 + (lane & 15), 0);
  }
  f32x4 acc[2][NSUB];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[b][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (g1 > g0)
    stream_two<NSUB, 4, GPT, PLANE, BD, BD>(d, d, st0, st1, g0, g1, rowp, xs, sx_region<NSUB, PLANE>(lds, a.RZ),
                                            lut_region<NSUB, PLANE>(lds, a.RZ, wave), acc, p0, p1);
  if (z_late<PLANE>() && epi) {
    __syncthreads();     // every wave is done with the staging area
    z_prologue<NSUB, 4>(a, false, a.zp_d, a.RZ, a.ks_stride_d, a.ks_d, zw, ch, zs);
    __syncthreads();
  }
  float *yp = a.ypart + (int64_t)split * a.P * a.H;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int row = (b ? st1 : st0) * 16 + (lane & 15);
    if (epi) {
      if (a.r > 0) lowrank_epi<NSUB>(d.U, a.r, a.Rp, row, zs, zw, acc[b], ub[b]);
      if (a.rs > 0) lowrank_epi<NSUB>(d.Us, a.rs, a.Rsp, row, zs + a.Rp, zw, acc[b]);
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * s + 4 * (lane >> 4) + i;
        if (m < ch.cnt) yp[(int64_t)(ch.base + m) * a.H + row] = acc[b][s][i];
      }
    }
  }
}

__device__ __forceinline__ uint16_t *dyn_lds() {
  extern __shared__ __attribute__((aligned(16))) uint16_t moeq_dyn_lds[];
  return moeq_dyn_lds;
}

// Chunk class by token tiles: NSUB = 1 when no chunk can exceed 16 tokens,
// else 2 (up to 32 tokens, the smaller chunks included: one launch fewer
// costs less than their idle MFMA rows).  One launch per call.
__device__ __forceinline__ int chunk_class(int nsub_max) { return nsub_max == 1 ? 1 : 2; }

// LDS bytes of one class: x staging, z rows (in the staging area for the
// bit-plane kernels), column sums, per-wave LUTs.
inline size_t stream_lds_bytes(bool plane, int nsub, int RZ) {
  const size_t nb = plane ? 1 : (nsub == 1 ? xs_bufs<1, false>() : 1);
  return nb * nsub * 16 * kXStride * 2 + (plane ? 0 : (size_t)nsub * 16 * 2 * RZ * 2) + nb * 8 * nsub * 16 * 4 +
         (plane ? (size_t)4 * 2 * kLutBlk * 2 : 0);
}

// gate/up: 256 threads; grid.x = max_chunks * (I / 64)
template <int NSUB, int GPT, bool PLANE>
__global__ void __launch_bounds__(256, NSUB == 1 ? 4 : 3) gateup_kernel(FfnArgs a) {
  static_assert(NSUB == 1 || NSUB == 2, "chunks hold at most 32 tokens");
  uint16_t *lds = dyn_lds();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_sg = a.I / 64;
  const int chunk = blockIdx.x / n_sg, sg = blockIdx.x % n_sg;
  Chunk ch;
  if (!find_chunk(a.offsets, a.E, chunk, &ch) || chunk_class(a.nsub_max) != NSUB) return;
  const int strip = 4 * sg + wave;
  const int bg = a.desc[3 * ch.e].bits, bu = a.desc[3 * ch.e + 1].bits;
  switch (bg * 4 + bu) {
    case 2 * 4 + 2: gateup_body<NSUB, GPT, PLANE, 2, 2>(a, ch, strip, lds); break;
    case 2 * 4 + 3: gateup_body<NSUB, GPT, PLANE, 2, 3>(a, ch, strip, lds); break;
    case 2 * 4 + 4: gateup_body<NSUB, GPT, PLANE, 2, 4>(a, ch, strip, lds); break;
    case 3 * 4 + 2: gateup_body<NSUB, GPT, PLANE, 3, 2>(a, ch, strip, lds); break;
    case 3 * 4 + 3: gateup_body<NSUB, GPT, PLANE, 3, 3>(a, ch, strip, lds); break;
    case 3 * 4 + 4: gateup_body<NSUB, GPT, PLANE, 3, 4>(a, ch, strip, lds); break;
    case 4 * 4 + 2: gateup_body<NSUB, GPT, PLANE, 4, 2>(a, ch, strip, lds); break;
    case 4 * 4 + 3: gateup_body<NSUB, GPT, PLANE, 4, 3>(a, ch, strip, lds); break;
    default: gateup_body<NSUB, GPT, PLANE, 4, 4>(a, ch, strip, lds); break;
  }
}

// down: 256 threads, 128 rows; grid.x = max_chunks * (H / 128) * splits
template <int NSUB, int GPT, bool PLANE>
__global__ void __launch_bounds__(256, NSUB == 1 ? 4 : 3) down_kernel(FfnArgs a) {
  static_assert(NSUB == 1 || NSUB == 2, "chunks hold at most 32 tokens");
  uint16_t *lds = dyn_lds();
  const int n_sg = a.H / 128;
  const int split = blockIdx.x % a.splits;
  const int rest = blockIdx.x / a.splits;
  const int chunk = rest / n_sg, sg = rest % n_sg;
  Chunk ch;
  if (!find_chunk(a.offsets, a.E, chunk, &ch) || chunk_class(a.nsub_max) != NSUB) return;
  switch (a.desc[3 * ch.e + 2].bits) {
    case 2: down_body<NSUB, GPT, PLANE, 2>(a, ch, sg, split, lds); break;
    case 3: down_body<NSUB, GPT, PLANE, 3>(a, ch, sg, split, lds); break;
    default: down_body<NSUB, GPT, PLANE, 4>(a, ch, sg, split, lds); break;
  }
}

// Launch helpers for one (GPT, PLANE) class, instantiated in the .hip files.
template <int GPT, bool PLANE>
void launch_gateup_class(const FfnArgs &a, int grid, hipStream_t s) {
  if (a.nsub_max == 1)
    hipLaunchKernelGGL((gateup_kernel<1, GPT, PLANE>), dim3(grid), dim3(256), stream_lds_bytes(PLANE, 1, a.RZ), s, a);
  else
    hipLaunchKernelGGL((gateup_kernel<2, GPT, PLANE>), dim3(grid), dim3(256), stream_lds_bytes(PLANE, 2, a.RZ), s, a);
}

template <int GPT, bool PLANE>
void launch_down_class(const FfnArgs &a, int grid, hipStream_t s) {
  if (a.nsub_max == 1)
    hipLaunchKernelGGL((down_kernel<1, GPT, PLANE>), dim3(grid), dim3(256), stream_lds_bytes(PLANE, 1, a.RZ), s, a);
  else
    hipLaunchKernelGGL((down_kernel<2, GPT, PLANE>), dim3(grid), dim3(256), stream_lds_bytes(PLANE, 2, a.RZ), s, a);
}

void launch_gateup_g128(const FfnArgs &a, int grid, hipStream_t s);
void launch_gateup_g64(const FfnArgs &a, int grid, hipStream_t s);
void launch_gateup_plane(const FfnArgs &a, int grid, hipStream_t s);
void launch_down_g128(const FfnArgs &a, int grid, hipStream_t s);
void launch_down_g64(const FfnArgs &a, int grid, hipStream_t s);
void launch_down_plane(const FfnArgs &a, int grid, hipStream_t s);

}  // namespace moeq
