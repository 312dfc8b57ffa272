// Tiled expert GEMMs for many tokens per expert (prefill).  Same operation
// as the weight-streaming kernels (PagedWeight review summary: one fused
// kernel over per-block variable bitwidths; MiLo / TileQ abstracts: the
// low-rank terms fused into the expert pass), organised for reuse instead
// of streaming:
//
//   - a workgroup computes a 128-token x 256-row output tile of one expert
//     (gate/up: 128 rows of I for both gate and up, so SwiGLU is formed in
//     registers; down: 256 rows of H);
//   - 4 waves, each owning 4 strips of 16 rows over all 128 tokens: 32
//     MFMA 16x16x32 tiles per 32-column step;
//   - K walks 128-column tiles; the activation tile (128 tokens x 128
//     columns, rows gathered by token for gate/up) is double-buffered in LDS
//     with one barrier per tile; each wave loads its strips' packed codes
//     and scales/zeros for the next tile straight into registers (the
//     packed layout already is the MFMA B-operand layout);
//   - INT codes decode to fp16 s*(c - z): exact (c - z) from the magic-bias
//     AND-OR and one packed FMA, then one packed multiply by the group's
//     fp16 scale (rounded once to fp16);
//   - workgroups are ordered token-tile-major and mapped so that the
//     workgroups of one token tile run on one XCD and share its L2.
#pragma once
#include "stream.hpp"

namespace moeq {

constexpr int kTM = kTiledM;           // tokens per token tile
constexpr int kTS = kTileK + 8;        // LDS row stride (halves) of a staged activation tile
constexpr int kTBuf = kTM * kTS;       // halves per activation buffer
constexpr size_t kTiledLdsBytes = (size_t)2 * kTBuf * 2;
#ifndef MOEQ_TILED_WAVES
#define MOEQ_TILED_WAVES 8
#endif
constexpr int kTiledWaves = MOEQ_TILED_WAVES;   // waves per workgroup: 4 (8 token tiles each) or 8 (4 each)

// Packed codes and metadata of one strip for one 128-column tile.
template <int B>
struct TTile {
  uint32_t w[B];
  uint32_t sc;   // fp16 scale of group gi in half gi
  uint32_t zz;   // zero of group gi in byte gi
};

// Address of dword e of tile t of strip s for lane l: the int_word_offset
// layout written as (uniform part) + l * (uniform lane stride), so that the
// full/ragged group choice is a scalar select.
template <int B>
__device__ __forceinline__ const uint8_t *tile_word_ptr(const uint8_t *codes, int s, int t, int e, int n_kt) {
  const int lane = threadIdx.x & 63;
  const int g4 = t >> 2, tl = t & 3;
  const int c = std::min(4, n_kt - 4 * g4);
  const uint64_t base = (uint64_t)s * n_kt * 256 * B + (uint64_t)g4 * 1024 * B;
  const int d = tl * B + e;
  const int ls = c == 4 ? 16 : c * 4 * B;
  const int ts = c == 4 ? (d >> 2) * 1024 + (d & 3) * 4 : tl * 4 * B + e * 4;
  return codes + base + ts + lane * ls;
}

template <int B, int GPT>
__device__ __forceinline__ void load_ttile(const BlockDesc &d, int strip, int t, int n_kt, TTile<B> &o) {
  const int lane = threadIdx.x & 63;
  if constexpr (B == 4) {
    const u32x4 v = gld<u32x4>(tile_word_ptr<4>(d.codes, strip, t, 0, n_kt));
    o.w[0] = v[0]; o.w[1] = v[1]; o.w[2] = v[2]; o.w[3] = v[3];
  } else if constexpr (B == 2) {
    const u32x2 v = gld<u32x2>(tile_word_ptr<2>(d.codes, strip, t, 0, n_kt));
    o.w[0] = v[0]; o.w[1] = v[1];
  } else {
#pragma unroll
    for (int e = 0; e < B; ++e) o.w[e] = gld<uint32_t>(tile_word_ptr<B>(d.codes, strip, t, e, n_kt));
  }
  const uint64_t mi = meta_index(strip, t, lane & 15, 0, n_kt, GPT);
  if constexpr (GPT == 1) {
    o.sc = gld<uint16_t>(d.scales + mi);
    o.zz = gld<uint8_t>(d.zeros + mi);
  } else {
    o.sc = gld<uint32_t>(d.scales + mi);
    o.zz = gld<uint16_t>(d.zeros + mi);
  }
}

// fp16 B operand s * (c - z) of step j of a tile.
template <int B, int GPT>
__device__ __forceinline__ f16x8 tdecode(const TTile<B> &tt, int j) {
  const int gi = GPT == 2 ? (j >> 1) : 0;
  PairConst pc[9];
  fill_pair_consts<B>(pc, (tt.zz >> (8 * gi)) & 0xffu);
  const f16 s = __builtin_bit_cast(f16, (uint16_t)(tt.sc >> (16 * gi)));
  const f16x2 s2 = {s, s};
  uint32_t p[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) p[v] = as_u32(as_h2(int_pair_cz<B>(tt.w, 4 * j + v, pc)) * s2);
  return pack_b(p[0], p[1], p[2], p[3]);
}

// Activation tile staging by the NW waves of the workgroup: thread tid moves
// rows (tid / 16) + 4 NW i, 16 B at column 8 (tid % 16), for i < 32 / NW.
// Row offsets are element offsets from the source base (gathered token rows
// of x, or contiguous rows of h).
template <int NW>
struct TStage {
  static constexpr int NP = 32 / NW;
  u32x4 v[NP];
};

template <int NW>
__device__ __forceinline__ void tstage_load(TStage<NW> &st, const uint16_t *src, const uint32_t *rowoff, int kt) {
  const int col = kt * kTileK + 8 * (threadIdx.x & 15);
#pragma unroll
  for (int i = 0; i < TStage<NW>::NP; ++i) st.v[i] = gld<u32x4>(src + rowoff[i] + col);
}

template <int NW>
__device__ __forceinline__ void tstage_store(const TStage<NW> &st, uint16_t *buf) {
  const int r0 = threadIdx.x >> 4, col = 8 * (threadIdx.x & 15);
#pragma unroll
  for (int i = 0; i < TStage<NW>::NP; ++i)
    *reinterpret_cast<u32x4 *>(buf + (r0 + 4 * NW * i) * kTS + col) = st.v[i];
}

__device__ __forceinline__ f16x8 tlds_a(const uint16_t *buf, int s, int j) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const f16x8 *>(buf + (16 * s + (lane & 15)) * kTS + 32 * j + 8 * (lane >> 4));
}

// The four strips of a wave: q = 0, 1 from block d0 (bits B0), q = 2, 3
// from block d1 (bits B1).
template <int B0, int B1>
struct TSet {
  TTile<B0> a0, a1;
  TTile<B1> b0, b1;
};

template <int B0, int B1, int GPT>
__device__ __forceinline__ void tset_load(TSet<B0, B1> &ts, const BlockDesc &d0, const BlockDesc &d1,
                                          const int *strips, int t, int n_kt) {
  load_ttile<B0, GPT>(d0, strips[0], t, n_kt, ts.a0);
  load_ttile<B0, GPT>(d0, strips[1], t, n_kt, ts.a1);
  load_ttile<B1, GPT>(d1, strips[2], t, n_kt, ts.b0);
  load_ttile<B1, GPT>(d1, strips[3], t, n_kt, ts.b1);
}

// One 128-column tile: NT token tiles (starting at token tile t0) x 4 strips.
template <int B0, int B1, int GPT, int NT>
__device__ __forceinline__ void tset_compute(const TSet<B0, B1> &ts, const uint16_t *buf, int t0,
                                             f32x4 (*acc)[NT]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x8 w0 = tdecode<B0, GPT>(ts.a0, j), w1 = tdecode<B0, GPT>(ts.a1, j);
    const f16x8 w2 = tdecode<B1, GPT>(ts.b0, j), w3 = tdecode<B1, GPT>(ts.b1, j);
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      const f16x8 av = tlds_a(buf, t0 + s, j);
      acc[0][s] = mfma16(av, w0, acc[0][s]);
      acc[1][s] = mfma16(av, w1, acc[1][s]);
      acc[2][s] = mfma16(av, w2, acc[2][s]);
      acc[3][s] = mfma16(av, w3, acc[3][s]);
    }
  }
}

// The K loop over all n_kt tiles, unrolled by two so that the register
// sets and LDS buffers of consecutive tiles alternate without copies.  The
// body has no branches: the prefetch after the last tile re-reads the last
// tile (its data is never used).
template <int B0, int B1, int GPT, int NW, int NT>
__device__ __forceinline__ void tiled_kloop(const BlockDesc &d0, const BlockDesc &d1, const int *strips, int n_kt,
                                            const uint16_t *src, const uint32_t *rowoff, uint16_t *lds, int t0,
                                            f32x4 (*acc)[NT]) {
  uint16_t *buf0 = lds, *buf1 = lds + kTBuf;
  TSet<B0, B1> s0, s1;
  TStage<NW> st;
  tstage_load<NW>(st, src, rowoff, 0);
  tset_load<B0, B1, GPT>(s0, d0, d1, strips, 0, n_kt);
  tstage_store<NW>(st, buf0);
  __syncthreads();
  int kt = 0;
#pragma unroll 1
  for (; kt + 2 <= n_kt; kt += 2) {
    tstage_load<NW>(st, src, rowoff, kt + 1);
    tset_load<B0, B1, GPT>(s1, d0, d1, strips, kt + 1, n_kt);
    tset_compute<B0, B1, GPT, NT>(s0, buf0, t0, acc);
    tstage_store<NW>(st, buf1);
    __syncthreads();
    const int kn = std::min(kt + 2, n_kt - 1);
    tstage_load<NW>(st, src, rowoff, kn);
    tset_load<B0, B1, GPT>(s0, d0, d1, strips, kn, n_kt);
    tset_compute<B0, B1, GPT, NT>(s1, buf1, t0, acc);
    tstage_store<NW>(st, buf0);
    __syncthreads();
  }
  if (kt < n_kt) {            // odd tile count: the last tile is in set 0 / buffer 0
    tset_compute<B0, B1, GPT, NT>(s0, buf0, t0, acc);
    __syncthreads();
  }
}

// Workgroup b of n (n a multiple of 8): workgroups are dealt to the 8 XCDs
// round-robin, so logical tile L = (b % 8) * (n / 8) + b / 8 gives each
// XCD a contiguous run of tiles.
__device__ __forceinline__ int xcd_tile(int b, int n) { return (b & 7) * (n >> 3) + (b >> 3); }

// Wave w of NW: strip group wn = w % 4, token tiles NT * (w / 4) + [0, NT)
// with NT = 32 / NW.
template <int NW>
struct TWave {
  static constexpr int NT = 32 / NW;
  int wn, t0;
  __device__ __forceinline__ TWave() {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wn = w & 3;
    t0 = NT * (w >> 2);
  }
};

template <int NW>
__device__ __forceinline__ void zero_acc(f32x4 (*acc)[32 / NW]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int s = 0; s < 32 / NW; ++s) acc[q][s] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// gate/up: strip group wn owns I rows nt*128 + 32 wn + [0, 32) of gate
// (q = 0, 1) and up (q = 2, 3).
template <int BG, int BU, int GPT, int NW>
__device__ __forceinline__ void tiled_gateup_body(const FfnArgs &a, const Chunk &ch, int nt, uint16_t *lds) {
  constexpr int NT = 32 / NW, NP = 32 / NW;
  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  const TWave<NW> w;
  const BlockDesc dg = a.desc[3 * ch.e], du = a.desc[3 * ch.e + 1];
  const int sg = nt * 8 + 2 * w.wn;
  const int strips[4] = {sg, sg + 1, sg, sg + 1};
  uint32_t rowoff[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int m = std::min((tid >> 4) + 4 * NW * i, ch.cnt - 1);
    rowoff[i] = (uint32_t)(a.sorted_pairs[ch.base + m] / a.k) * (uint32_t)a.H;
  }
  f32x4 acc[4][NT];
  zero_acc<NW>(acc);
  tiled_kloop<BG, BU, GPT, NW, NT>(dg, du, strips, a.H / kTileK, a.x, rowoff, lds, w.t0, acc);
  // the loop ends with a barrier: the activation buffers are free
  if (a.comp_on) {
    uint16_t *zs = lds;
    const int zw = 2 * a.RZ;
    z_prologue<8, NW>(a.zp_gu, zw, a.ks_stride_gu, a.ks_gu, zw, ch, zs);
    __syncthreads();
    const uint16_t *zw0 = zs + 16 * w.t0 * zw;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b = q >> 1;
      const BlockDesc &d = b ? du : dg;
      const int row = strips[q] * 16 + (lane & 15);
      if (a.r > 0) lowrank_epi<NT>(d.U, a.r, a.Rp, row, zw0 + b * a.RZ, zw, acc[q]);
      if (a.rs > 0) lowrank_epi<NT>(d.Us, a.rs, a.Rsp, row, zw0 + b * a.RZ + a.Rp, zw, acc[q]);
    }
    __syncthreads();
  }
  // h = SiLU(gate) * up into LDS [128 tokens][128 columns], then coalesced rows
  uint16_t *hs = lds;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int col = 32 * w.wn + 16 * g + (lane & 15);
#pragma unroll
    for (int s = 0; s < NT; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gv = acc[g][s][i], uv = acc[2 + g][s][i];
        const float hv = gv / (1.0f + __expf(-gv)) * uv;
        hs[(16 * (w.t0 + s) + 4 * (lane >> 4) + i) * kTS + col] = __builtin_bit_cast(uint16_t, (f16)hv);
      }
    }
  }
  __syncthreads();
  const int c8 = 8 * (tid & 15);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = (tid >> 4) + 4 * NW * i;
    if (r < ch.cnt)
      *reinterpret_cast<u32x4 *>(a.h + (int64_t)(ch.base + r) * a.I + nt * kTileK + c8) =
          *reinterpret_cast<const u32x4 *>(hs + r * kTS + c8);
  }
}

// down: strip group wn owns H rows nt*256 + 64 wn + [0, 64).
template <int BD, int GPT, int NW>
__device__ __forceinline__ void tiled_down_body(const FfnArgs &a, const Chunk &ch, int nt, uint16_t *lds) {
  constexpr int NT = 32 / NW, NP = 32 / NW;
  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  const TWave<NW> w;
  const BlockDesc d = a.desc[3 * ch.e + 2];
  const int s0 = nt * 16 + 4 * w.wn;
  const int strips[4] = {s0, s0 + 1, s0 + 2, s0 + 3};
  uint32_t rowoff[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int m = std::min((tid >> 4) + 4 * NW * i, ch.cnt - 1);
    rowoff[i] = (uint32_t)(ch.base + m) * (uint32_t)a.I;
  }
  f32x4 acc[4][NT];
  zero_acc<NW>(acc);
  tiled_kloop<BD, BD, GPT, NW, NT>(d, d, strips, a.I / kTileK, a.h, rowoff, lds, w.t0, acc);
  if (a.comp_on) {
    uint16_t *zs = lds;
    z_prologue<8, NW>(a.zp_d, a.RZ, a.ks_stride_d, a.ks_d, a.RZ, ch, zs);
    __syncthreads();
    const uint16_t *zw0 = zs + 16 * w.t0 * a.RZ;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = strips[q] * 16 + (lane & 15);
      if (a.r > 0) lowrank_epi<NT>(d.U, a.r, a.Rp, row, zw0, a.RZ, acc[q]);
      if (a.rs > 0) lowrank_epi<NT>(d.Us, a.rs, a.Rsp, row, zw0 + a.Rp, a.RZ, acc[q]);
    }
  }
  float *yp = a.ypart;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = strips[q] * 16 + (lane & 15);
#pragma unroll
    for (int s = 0; s < NT; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * (w.t0 + s) + 4 * (lane >> 4) + i;
        if (m < ch.cnt) yp[(int64_t)(ch.base + m) * a.H + row] = acc[q][s][i];
      }
    }
  }
}

// grid.x = (upper bound of token tiles) * (I / 128), rounded up to 8
template <int GPT, int NW>
__global__ void __launch_bounds__(64 * NW, 1) tiled_gateup_kernel(FfnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t tl_lds[];
  const int n_nt = a.I / kTileK;
  const int L = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = L / n_nt, nt = L % n_nt;
  Chunk ch;
  if (!find_chunk<kTM>(a.offsets, a.E, mt, &ch)) return;
  const int bg = a.desc[3 * ch.e].bits, bu = a.desc[3 * ch.e + 1].bits;
  switch (bg * 4 + bu) {
    case 2 * 4 + 2: tiled_gateup_body<2, 2, GPT, NW>(a, ch, nt, tl_lds); break;
    case 2 * 4 + 3: tiled_gateup_body<2, 3, GPT, NW>(a, ch, nt, tl_lds); break;
    case 2 * 4 + 4: tiled_gateup_body<2, 4, GPT, NW>(a, ch, nt, tl_lds); break;
    case 3 * 4 + 2: tiled_gateup_body<3, 2, GPT, NW>(a, ch, nt, tl_lds); break;
    case 3 * 4 + 3: tiled_gateup_body<3, 3, GPT, NW>(a, ch, nt, tl_lds); break;
    case 3 * 4 + 4: tiled_gateup_body<3, 4, GPT, NW>(a, ch, nt, tl_lds); break;
    case 4 * 4 + 2: tiled_gateup_body<4, 2, GPT, NW>(a, ch, nt, tl_lds); break;
    case 4 * 4 + 3: tiled_gateup_body<4, 3, GPT, NW>(a, ch, nt, tl_lds); break;
    default: tiled_gateup_body<4, 4, GPT, NW>(a, ch, nt, tl_lds); break;
  }
}

// grid.x = (upper bound of token tiles) * (H / 256), rounded up to 8
template <int GPT, int NW>
__global__ void __launch_bounds__(64 * NW, 1) tiled_down_kernel(FfnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t tl_lds[];
  const int n_nt = a.H / 256;
  const int L = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = L / n_nt, nt = L % n_nt;
  Chunk ch;
  if (!find_chunk<kTM>(a.offsets, a.E, mt, &ch)) return;
  switch (a.desc[3 * ch.e + 2].bits) {
    case 2: tiled_down_body<2, GPT, NW>(a, ch, nt, tl_lds); break;
    case 3: tiled_down_body<3, GPT, NW>(a, ch, nt, tl_lds); break;
    default: tiled_down_body<4, GPT, NW>(a, ch, nt, tl_lds); break;
  }
}

}  // namespace moeq
