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
//   - K walks 128-column tiles through three LDS stages filled by LDS-DMA
//     loads two tiles ahead (activation rows gathered by token for gate/up,
//     XOR-swizzled; the packed codes, whose layout already is the MFMA
//     B-operand layout per lane), one barrier per tile;
//   - INT codes decode to fp16 s*(c - z): exact (c - z) from the magic-bias
//     AND-OR and one packed FMA, then one packed multiply by the group's
//     fp16 scale (rounded once to fp16);
//   - workgroups are ordered token-tile-major and mapped so that the
//     workgroups of one token tile run on one XCD and share its L2.
#pragma once
#include "stream.hpp"

namespace moeq {

constexpr int kTM = kTiledM;           // tokens per token tile
constexpr int kTS = kTileK + 8;        // LDS row stride (halves) of the staged h tile
constexpr int kTiledWaves = 4;   // waves per workgroup (8 token tiles x 4 strips each)

// Packed codes and metadata of one strip for one 128-column tile.
template <int B>
struct TTile {
  uint32_t w[B];
  uint32_t sc;   // fp16 scale of group gi in half gi
  uint32_t zz;   // zero of group gi in byte gi
};

// Offset of dword e of tile t of strip s for lane l in an INT code region:
// the int_word_offset layout written as (uniform part) + l * (uniform lane
// stride), so that the full/ragged group choice is a scalar select.
struct WordOff {
  uint32_t uni, lane;
};
template <int B>
__device__ __forceinline__ WordOff tile_word_off(int s, int t, int e, int n_kt) {
  const int lane = threadIdx.x & 63;
  const int g4 = t >> 2, tl = t & 3;
  const int c = std::min(4, n_kt - 4 * g4);
  const uint32_t base = (uint32_t)s * n_kt * 256 * B + (uint32_t)g4 * 1024 * B;
  const int d = tl * B + e;
  const int ls = c == 4 ? 16 : c * 4 * B;
  const int ts = c == 4 ? (d >> 2) * 1024 + (d & 3) * 4 : tl * 4 * B + e * 4;
  return WordOff{base + (uint32_t)ts, (uint32_t)(lane * ls)};
}

// Bytes of an INT block's code region (b dwords per lane per tile).
__device__ __forceinline__ uint32_t code_region_bytes(const BlockDesc &d) {
  return (uint32_t)(d.N / kStripRows) * (uint32_t)(d.K / kTileK) * 256u * (uint32_t)d.bits;
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

// ---- LDS stages.  A stage holds one 128-column tile: the activation tile
// (128 token rows x 256 B, 16-byte slots XOR-swizzled by row so that the
// MFMA operand reads are bank-conflict free), the packed codes of the
// workgroup's 16 strips (1 KiB each) and their scales and zeros.  All of
// it is written by the LDS forms of the loads (activations and codes:
// buffer_load ... lds against buffer resources, i.e. a scalar base plus a
// 32-bit lane offset; scales and zeros: global_load_lds): the data never
// occupies registers, so tiles are fetched two ahead of the
// MFMAs through three stages, and the only memory counter the loop waits
// on is the one for these transfers (explicit waits: the compiler does not
// track DMA writes into LDS).
constexpr int kTABytes = kTM * 256;
constexpr int kTBBytes = 16 * 1024;
constexpr int kTMetaBytes = 4 * 512;                  // per wave: 64 lanes x 2 dword slots
constexpr int kTStageBytes = kTABytes + kTBBytes + kTMetaBytes;
constexpr int kTStages = 3;

// DMA operations per strip per tile: one 16-byte transfer for 4-bit codes,
// else one 4-byte transfer per code dword.
__device__ __forceinline__ constexpr int dma_ops(int B) { return B == 4 ? 1 : B; }

template <int B>
__device__ __forceinline__ void dma_codes(__amdgpu_buffer_rsrc_t codes, int strip, int t, int n_kt, uint8_t *dst) {
  if constexpr (B == 4) {
    const WordOff o = tile_word_off<4>(strip, t, 0, n_kt);
    lds_dma_buf<16>(codes, o.lane, o.uni, dst);
  } else {
#pragma unroll
    for (int e = 0; e < B; ++e) {
      const WordOff o = tile_word_off<B>(strip, t, e, n_kt);
      lds_dma_buf<4>(codes, o.lane, o.uni, dst + 256 * e);
    }
  }
}

template <int B>
__device__ __forceinline__ void lds_codes(const uint8_t *src, TTile<B> &tt) {
  const int lane = threadIdx.x & 63;
  if constexpr (B == 4) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(src + 16 * lane);
    tt.w[0] = v[0]; tt.w[1] = v[1]; tt.w[2] = v[2]; tt.w[3] = v[3];
  } else {
#pragma unroll
    for (int e = 0; e < B; ++e) tt.w[e] = *reinterpret_cast<const uint32_t *>(src + 256 * e + 4 * lane);
  }
}

// Operand A of token tile s, step j from the swizzled activation tile.
__device__ __forceinline__ f16x8 tlds_a(const uint8_t *abuf, int s, int j) {
  const int lane = threadIdx.x & 63;
  const int row = 16 * s + (lane & 15), c = 4 * j + (lane >> 4);
  return *reinterpret_cast<const f16x8 *>(abuf + row * 256 + 16 * (c ^ (row & 15)));
}

// The strips of wave w: q = 0, 1 from block d0 (bits B0), q = 2, 3 from d1
// (bits B1); their codes sit at 1 KiB slots 4 w + q of the stage, their
// scales/zeros in lanes 16 q .. 16 q + 15 of the wave's metadata slots.
template <int B0, int B1, int GPT>
struct TKLoop {
  static constexpr int kDma = 8 + 2 * dma_ops(B0) + 2 * dma_ops(B1) + 2;   // DMA ops per tile per wave
  const BlockDesc &d0, &d1;
  const int *strips;
  int n_kt, wave;
  const uint32_t *rowoff;
  uint8_t *lds;
  __amdgpu_buffer_rsrc_t ra, rc0, rc1;   // activations, codes of d0 and of d1

  __device__ __forceinline__ uint8_t *stage(int st) const { return lds + st * kTStageBytes; }

  // tile t into stage st: the wave's 8 KiB share of the activation tile,
  // its strips' codes, scales and zeros
  __device__ __forceinline__ void issue(int t, int st) const {
    const int lane = threadIdx.x & 63;
    uint8_t *a = stage(st);
    // buffer loads: uniform tile offset + loop-invariant 32-bit lane offset
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 32 * wave + 4 * i + (lane >> 4);
      const uint32_t c = (uint32_t)((lane & 15) ^ (row & 15));
      lds_dma_buf<16>(ra, 2u * (rowoff[i] + 8u * c), (uint32_t)t * (kTileK * 2), a + (32 * wave + 4 * i) * 256);
    }
    uint8_t *b = stage(st) + kTABytes + 4 * wave * 1024;
    dma_codes<B0>(rc0, strips[0], t, n_kt, b);
    dma_codes<B0>(rc0, strips[1], t, n_kt, b + 1024);
    dma_codes<B1>(rc1, strips[2], t, n_kt, b + 2048);
    dma_codes<B1>(rc1, strips[3], t, n_kt, b + 3072);
    // lane l: strip q = l / 16, row l % 16
    const int q = lane >> 4;
    const BlockDesc &dq = q < 2 ? d0 : d1;
    const uint64_t mi = meta_index(strips[q], t, lane & 15, 0, n_kt, GPT);
    uint8_t *m = stage(st) + kTABytes + kTBBytes + wave * 512;
    lds_dma<2 * GPT>(dq.scales + mi, m);       // dword slot per lane
    lds_dma<GPT>(dq.zeros + mi, m + 256);      // zero-extended dword slot per lane
  }

  template <int NT>
  __device__ __forceinline__ void compute(int st, f32x4 (*acc)[NT]) const {
    const int lane = threadIdx.x & 63;
    const uint8_t *a = stage(st);
    const uint8_t *b = stage(st) + kTABytes + 4 * wave * 1024;
    const uint8_t *m = stage(st) + kTABytes + kTBBytes + wave * 512;
    TTile<B0> t0, t1;
    TTile<B1> t2, t3;
    lds_codes<B0>(b, t0);
    lds_codes<B0>(b + 1024, t1);
    lds_codes<B1>(b + 2048, t2);
    lds_codes<B1>(b + 3072, t3);
    const int r = lane & 15;
    const uint32_t *sc = reinterpret_cast<const uint32_t *>(m);
    const uint32_t *zz = reinterpret_cast<const uint32_t *>(m + 256);
    t0.sc = sc[r]; t1.sc = sc[16 + r]; t2.sc = sc[32 + r]; t3.sc = sc[48 + r];
    t0.zz = zz[r]; t1.zz = zz[16 + r]; t2.zz = zz[32 + r]; t3.zz = zz[48 + r];
    // activation fragments double-buffered across steps: step j + 1's NT
    // reads are in flight while step j is decoded and multiplied
    f16x8 av[2][NT];
#pragma unroll
    for (int s = 0; s < NT; ++s) av[0][s] = tlds_a(a, s, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < 3) {
#pragma unroll
        for (int s = 0; s < NT; ++s) av[(j + 1) & 1][s] = tlds_a(a, s, j + 1);
      }
      const f16x8 w0 = tdecode<B0, GPT>(t0, j), w1 = tdecode<B0, GPT>(t1, j);
      const f16x8 w2 = tdecode<B1, GPT>(t2, j), w3 = tdecode<B1, GPT>(t3, j);
#pragma unroll
      for (int s = 0; s < NT; ++s) {
        acc[0][s] = mfma16(av[j & 1][s], w0, acc[0][s]);
        acc[1][s] = mfma16(av[j & 1][s], w1, acc[1][s]);
        acc[2][s] = mfma16(av[j & 1][s], w2, acc[2][s]);
        acc[3][s] = mfma16(av[j & 1][s], w3, acc[3][s]);
      }
    }
  }

  // one K tile: wait for its stage (the next tile's transfers may stay in
  // flight), barrier (every wave's transfers done; every wave has finished
  // reading the stage of tile t - 1), queue tile t + 2 into that stage,
  // multiply
  template <int ST, int NT>
  __device__ __forceinline__ void step(int t, f32x4 (*acc)[NT]) const {
    vm_wait<kDma>();
    __builtin_amdgcn_s_barrier();
    issue(std::min(t + 2, n_kt - 1), (ST + 2) % 3);
    compute<NT>(ST, acc);
  }

  template <int NT>
  __device__ __forceinline__ void run(f32x4 (*acc)[NT]) const {
    issue(0, 0);
    issue(std::min(1, n_kt - 1), 1);
    int kt = 0;
#pragma unroll 1
    for (; kt + 3 <= n_kt; kt += 3) {
      step<0, NT>(kt, acc);
      step<1, NT>(kt + 1, acc);
      step<2, NT>(kt + 2, acc);
    }
    if (kt < n_kt) step<0, NT>(kt, acc);
    if (kt + 1 < n_kt) step<1, NT>(kt + 1, acc);
    // the queued re-reads of the last tile land before the LDS is reused
    vm_wait<0>();
    __syncthreads();
  }
};

// Workgroup b of n (n a multiple of 8): workgroups are dealt to the 8 XCDs
// round-robin, so logical tile L = (b % 8) * (n / 8) + b / 8 gives each
// XCD a contiguous run of tiles.
__device__ __forceinline__ int xcd_tile(int b, int n) { return (b & 7) * (n >> 3) + (b >> 3); }

// gate/up: wave w owns I rows nt*128 + 32 w + [0, 32) of gate (q = 0, 1)
// and up (q = 2, 3), for all 128 tokens of the tile.
template <int BG, int BU, int GPT>
__device__ __forceinline__ void tiled_gateup_body(const FfnArgs &a, const Chunk &ch, int nt, uint8_t *lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BlockDesc dg = a.desc[3 * ch.e], du = a.desc[3 * ch.e + 1];
  const int sg = nt * 8 + 2 * wave;
  const int strips[4] = {sg, sg + 1, sg, sg + 1};
  uint32_t rowoff[8];          // activation rows this lane moves: 32 w + 4 i + lane / 16
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = std::min(32 * wave + 4 * i + (lane >> 4), ch.cnt - 1);
    rowoff[i] = (uint32_t)(a.sorted_pairs[ch.base + m] / a.k) * (uint32_t)a.H;
  }
  f32x4 acc[4][8];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[q][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  const TKLoop<BG, BU, GPT> kl{dg,
                               du,
                               strips,
                               a.H / kTileK,
                               wave,
                               rowoff,
                               lds,
                               make_rsrc(a.x, (uint32_t)a.T * (uint32_t)a.H * 2u),
                               make_rsrc(dg.codes, code_region_bytes(dg)),
                               make_rsrc(du.codes, code_region_bytes(du))};
  // the low-rank epilogue's inputs (z rows for up to 64 columns from one
  // partial, and the first U operands) are requested before the K walk, so
  // the epilogue does not wait for memory
  const int zw = 2 * a.RZ;
  const bool zpre = a.comp_on && a.ks_gu == 1 && zw <= 64;
  ZPre<8, 4, 8> zp;
  if (zpre) z_preload<8, 4, 8>(a.zp_gu, zw, zw, ch, zp);
  f16x8 ub[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    ub[q] = a.comp_on && a.r > 0 ? lowrank_bop((q >> 1) ? du.U : dg.U, a.r, strips[q] * 16 + (lane & 15), 0)
                                 : pack_b(0, 0, 0, 0);
  kl.template run<8>(acc);
  uint16_t *l16 = reinterpret_cast<uint16_t *>(lds);
  if (a.comp_on) {
    uint16_t *zs = l16;
    if (zpre) z_store<8, 4, 8>(zp, zw, zs);
    else z_prologue<8, 4>(a.zp_gu, zw, a.ks_stride_gu, a.ks_gu, zw, ch, zs);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b = q >> 1;
      const BlockDesc &d = b ? du : dg;
      const int row = strips[q] * 16 + (lane & 15);
      if (a.r > 0) lowrank_epi<8>(d.U, a.r, a.Rp, row, zs + b * a.RZ, zw, acc[q], ub[q]);
      if (a.rs > 0) lowrank_epi<8>(d.Us, a.rs, a.Rsp, row, zs + b * a.RZ + a.Rp, zw, acc[q]);
    }
    __syncthreads();
  }
  // h = SiLU(gate) * up into LDS [128 tokens][128 columns], then coalesced rows
  uint16_t *hs = l16;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int col = 32 * wave + 16 * g + (lane & 15);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gv = acc[g][s][i], uv = acc[2 + g][s][i];
        const float hv = gv / (1.0f + __expf(-gv)) * uv;
        hs[(16 * s + 4 * (lane >> 4) + i) * kTS + col] = __builtin_bit_cast(uint16_t, (f16)hv);
      }
    }
  }
  __syncthreads();
  const int tid = threadIdx.x, c8 = 8 * (tid & 15);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 4) + 16 * i;
    if (r < ch.cnt)
      *reinterpret_cast<u32x4 *>(a.h + (int64_t)(ch.base + r) * a.I + nt * kTileK + c8) =
          *reinterpret_cast<const u32x4 *>(hs + r * kTS + c8);
  }
}

// down: wave w owns H rows nt*256 + 64 w + [0, 64).
template <int BD, int GPT>
__device__ __forceinline__ void tiled_down_body(const FfnArgs &a, const Chunk &ch, int nt, uint8_t *lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BlockDesc d = a.desc[3 * ch.e + 2];
  const int s0 = nt * 16 + 4 * wave;
  const int strips[4] = {s0, s0 + 1, s0 + 2, s0 + 3};
  uint32_t rowoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = std::min(32 * wave + 4 * i + (lane >> 4), ch.cnt - 1);
    rowoff[i] = (uint32_t)(ch.base + m) * (uint32_t)a.I;
  }
  f32x4 acc[4][8];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[q][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(d.codes, code_region_bytes(d));
  const TKLoop<BD, BD, GPT> kl{d, d, strips, a.I / kTileK, wave, rowoff, lds,
                               make_rsrc(a.h, (uint32_t)a.P * (uint32_t)a.I * 2u), rc, rc};
  kl.template run<8>(acc);
  if (a.comp_on) {
    uint16_t *zs = reinterpret_cast<uint16_t *>(lds);
    z_prologue<8, 4>(a.zp_d, a.RZ, a.ks_stride_d, a.ks_d, a.RZ, ch, zs);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = strips[q] * 16 + (lane & 15);
      if (a.r > 0) lowrank_epi<8>(d.U, a.r, a.Rp, row, zs, a.RZ, acc[q]);
      if (a.rs > 0) lowrank_epi<8>(d.Us, a.rs, a.Rsp, row, zs + a.Rp, a.RZ, acc[q]);
    }
  }
  float *yp = a.ypart;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = strips[q] * 16 + (lane & 15);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * s + 4 * (lane >> 4) + i;
        if (m < ch.cnt) yp[(int64_t)(ch.base + m) * a.H + row] = acc[q][s][i];
      }
    }
  }
}

// grid.x = (upper bound of token tiles) * (I / 128), rounded up to 8
template <int GPT>
__global__ void __launch_bounds__(256, 1) tiled_gateup_kernel(FfnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t tl_lds[];
  const int n_nt = a.I / kTileK;
  const int L = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = L / n_nt, nt = L % n_nt;
  Chunk ch;
  if (!find_chunk<kTM>(a.offsets, a.E, mt, &ch)) return;
  const int bg = a.desc[3 * ch.e].bits, bu = a.desc[3 * ch.e + 1].bits;
  switch (bg * 4 + bu) {
    case 2 * 4 + 2: tiled_gateup_body<2, 2, GPT>(a, ch, nt, tl_lds); break;
    case 2 * 4 + 3: tiled_gateup_body<2, 3, GPT>(a, ch, nt, tl_lds); break;
    case 2 * 4 + 4: tiled_gateup_body<2, 4, GPT>(a, ch, nt, tl_lds); break;
    case 3 * 4 + 2: tiled_gateup_body<3, 2, GPT>(a, ch, nt, tl_lds); break;
    case 3 * 4 + 3: tiled_gateup_body<3, 3, GPT>(a, ch, nt, tl_lds); break;
    case 3 * 4 + 4: tiled_gateup_body<3, 4, GPT>(a, ch, nt, tl_lds); break;
    case 4 * 4 + 2: tiled_gateup_body<4, 2, GPT>(a, ch, nt, tl_lds); break;
    case 4 * 4 + 3: tiled_gateup_body<4, 3, GPT>(a, ch, nt, tl_lds); break;
    default: tiled_gateup_body<4, 4, GPT>(a, ch, nt, tl_lds); break;
  }
}

// grid.x = (upper bound of token tiles) * (H / 256), rounded up to 8
template <int GPT>
__global__ void __launch_bounds__(256, 1) tiled_down_kernel(FfnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t tl_lds[];
  const int n_nt = a.H / 256;
  const int L = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = L / n_nt, nt = L % n_nt;
  Chunk ch;
  if (!find_chunk<kTM>(a.offsets, a.E, mt, &ch)) return;
  switch (a.desc[3 * ch.e + 2].bits) {
    case 2: tiled_down_body<2, GPT>(a, ch, nt, tl_lds); break;
    case 3: tiled_down_body<3, GPT>(a, ch, nt, tl_lds); break;
    default: tiled_down_body<4, GPT>(a, ch, nt, tl_lds); break;
  }
}

constexpr size_t kTiledLdsBytes = (size_t)kTStages * kTStageBytes;

}  // namespace moeq
