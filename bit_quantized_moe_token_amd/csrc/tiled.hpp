// Tiled expert GEMMs for many tokens per expert (prefill).  Same operation
// as the weight-streaming kernels (PagedWeight review summary: one fused
// kernel over per-block variable bitwidths; MiLo / TileQ abstracts: the
// low-rank terms fused into the expert pass), organised for reuse instead
// of streaming:
//
//   - a workgroup computes a 128-token x 256-row output tile of one expert
//     (gate/up: 128 rows of I for both gate and up, so SwiGLU is formed in
//     registers; down: 256 rows of H);
//   - 8 waves (two per SIMD, so that one wave's MFMAs run while the other
//     decodes or waits), each owning 2 strips of 16 rows over all 128
//     tokens: 16 MFMA 16x16x32 tiles per 32-column step;
//   - K walks 128-column tiles through three LDS stages filled by LDS-DMA
//     loads issued three tiles ahead (activation rows gathered by token
//     for gate/up, XOR-swizzled; the packed codes, whose layout already is
//     the MFMA B-operand layout per lane), one barrier per tile; within a
//     tile the next 32-column step's activation reads and weight decode
//     are spread between the current step's MFMAs;
//   - INT codes decode to fp16 s*(c - z): exact (c - z) from the magic-bias
//     AND-OR and one packed FMA, then one packed multiply by the group's
//     fp16 scale (rounded once to fp16);
//   - workgroups are ordered token-tile-major and mapped so that the
//     workgroups of one token tile run on one XCD and share its L2.
#pragma once
#include "stream.hpp"

namespace moeq {

constexpr int kTM = kTiledM;           // tokens per token tile
constexpr int kH32S = kTileK + 4;      // LDS row stride (floats) of the staged fp32 h tile
constexpr int kTiledWaves = 8;   // waves per workgroup (8 token tiles x 2 strips each)

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

// Bit-plane strip of one 128-column tile: the top q planes (one dword per
// plane; pl[u] = plane 3 - u, as plane_sel expects) and the lane's row LUT
// byte-split for the permute lookups (the 2^q low bytes in 2^q / 4 dwords,
// then the high bytes).  The LUT group is the tile (128 columns).
template <int Q>
struct PTile {
  uint32_t w[Q];
  uint32_t L[1 << (Q - 1)];
};

template <int B, bool PLANE>
struct TileOf {
  using type = TTile<B>;
};
template <int Q>
struct TileOf<Q, true> {
  using type = PTile<Q>;
};

// ---- LDS stages.  A stage holds one 128-column tile: the activation tile
// (128 token rows x 256 B, 16-byte slots XOR-swizzled by row so that the
// MFMA operand reads are bank-conflict free), the packed codes of the
// workgroup's 16 strips (1 KiB each) and their scales and zeros (a
// 512-byte slot per wave).  All of it is written by the LDS forms of the
// loads (activations and codes: buffer_load ... lds against buffer
// resources, i.e. a scalar base plus a 32-bit lane offset; scales and
// zeros: global_load_lds): the data never occupies registers, and the only
// memory counter the loop waits on is the one for these transfers
// (explicit waits: the compiler does not track DMA writes into LDS).
// Staging the same loads through registers (buffer loads, then LDS
// stores) measured slower.
// Bit-plane layers use the same stage with a 1 KiB slot per wave for the
// two strips' LUTs (16 rows x 2^q fp16, up to 512 bytes per strip) in place
// of the scales and zeros; that leaves room for two stages, not three.
constexpr int kTABytes = kTM * 256;
constexpr int kTBBytes = 16 * 1024;
template <bool PLANE>
struct TStages {
  static constexpr int kMeta = PLANE ? 1024 : 512;   // per wave (INT: 64 lanes x 2 dword slots)
  static constexpr int kBytes = kTABytes + kTBBytes + kTiledWaves * kMeta;
  static constexpr int kN = PLANE ? 2 : 3;
  static constexpr size_t kLds = (size_t)kN * kBytes;
  // dynamic LDS of a gate/up launch: the stages, then the rows' x
  // exponents and pair ids
  static constexpr size_t kLaunchGU = kLds + 2 * kTM * 4;
};
static_assert(TStages<false>::kLaunchGU <= 160 * 1024 && TStages<true>::kLaunchGU <= 160 * 1024, "LDS");

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

// Bit-plane codes: one 4-byte transfer per plane; plane u of lane l of
// tile t sits at u * plane_bytes + code_offset(strip, t, l, n_kt, 4).
template <int Q>
__device__ __forceinline__ void dma_planes(__amdgpu_buffer_rsrc_t codes, uint32_t plane_bytes, int strip, int t,
                                           int n_kt, uint8_t *dst) {
  const int lane = threadIdx.x & 63;
  const int g4 = t >> 2, tl = t & 3;
  const int c = std::min(4, n_kt - 4 * g4);
  const uint32_t uni = (uint32_t)strip * n_kt * 256 + (uint32_t)g4 * 1024 + (uint32_t)tl * 4;
#pragma unroll
  for (int u = 0; u < Q; ++u) lds_dma_buf<4>(codes, (uint32_t)(lane * c * 4), uni + (uint32_t)u * plane_bytes, dst + 256 * u);
}

template <int Q>
__device__ __forceinline__ void lds_planes(const uint8_t *src, PTile<Q> &tt) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < Q; ++u) tt.w[u] = *reinterpret_cast<const uint32_t *>(src + 256 * u + 4 * lane);
}

// The lane's row LUT (row lane % 16 of a strip's 16 x 2^q table at src),
// byte-split.
template <int Q>
__device__ __forceinline__ void lds_lut(const uint8_t *src, PTile<Q> &tt) {
  constexpr int NQ = 1 << Q;
  const uint8_t *row = src + (threadIdx.x & 15) * 2 * NQ;
  uint32_t v[NQ / 2];
  if constexpr (Q == 2) {
    const u32x2 a = *reinterpret_cast<const u32x2 *>(row);
    v[0] = a[0]; v[1] = a[1];
  } else {
#pragma unroll
    for (int i = 0; i < NQ / 8; ++i) {
      const u32x4 a = *reinterpret_cast<const u32x4 *>(row + 16 * i);
      v[4 * i] = a[0]; v[4 * i + 1] = a[1]; v[4 * i + 2] = a[2]; v[4 * i + 3] = a[3];
    }
  }
#pragma unroll
  for (int m = 0; m < NQ / 4; ++m) {
    tt.L[m] = __builtin_amdgcn_perm(v[2 * m + 1], v[2 * m], 0x06040200u);
    tt.L[NQ / 4 + m] = __builtin_amdgcn_perm(v[2 * m + 1], v[2 * m], 0x07050301u);
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

// The strips of wave w: q = 0 from block d0 (bits B0), q = 1 from d1 (bits
// B1); their codes sit at 1 KiB slots 2 w + q of the stage, their scales
// and zeros in lanes 16 q .. 16 q + 15 of the wave's metadata slots (lanes
// 32 .. 63 repeat lanes 0 .. 31).  Bit-plane (PLANE; B0, B1 the committed
// q): plane u of a strip at 256 u of its slot, the strips' LUTs at 0 and
// 512 of the wave's metadata slot (lanes 0 .. 31 move strip 0's table,
// 32 .. 63 strip 1's, 16 bytes each).
template <int B0, int B1, int GPT, bool PLANE = false>
struct TKLoop {
  using St = TStages<PLANE>;
  using Tile0 = typename TileOf<B0, PLANE>::type;
  using Tile1 = typename TileOf<B1, PLANE>::type;
  // DMA ops per tile per wave
  static constexpr int kDma = PLANE ? 4 + B0 + B1 + 1 : 4 + dma_ops(B0) + dma_ops(B1) + 2;
  const BlockDesc &d0, &d1;
  const int *strips;
  int n_kt, wave;
  const uint32_t *rowoff;
  uint8_t *lds;
  __amdgpu_buffer_rsrc_t ra, rc0, rc1;   // activations, codes of d0 and of d1

  // tile t into the stage at byte offset sb: the wave's 4 KiB share of the
  // activation tile (rows 16 w .. 16 w + 15), its strips' codes, scales and
  // zeros
  __device__ __forceinline__ void issue(int t, uint32_t sb) const {
    const int lane = threadIdx.x & 63;
    uint8_t *a = lds + sb;
    // buffer loads: uniform tile offset + loop-invariant 32-bit lane offset
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * i + (lane >> 4);
      const uint32_t c = (uint32_t)((lane & 15) ^ (row & 15));
      lds_dma_buf<16>(ra, 2u * (rowoff[i] + 8u * c), (uint32_t)t * (kTileK * 2), a + (16 * wave + 4 * i) * 256);
    }
    uint8_t *b = a + kTABytes + 2 * wave * 1024;
    if constexpr (PLANE) {
      dma_planes<B0>(rc0, (uint32_t)d0.plane_bytes, strips[0], t, n_kt, b);
      dma_planes<B1>(rc1, (uint32_t)d1.plane_bytes, strips[1], t, n_kt, b + 1024);
      // strip q's table: 16 rows x 2^q fp16 = 2 * 2^q 16-byte pieces
      const int q = lane >> 5, i = lane & 31;
      const int nq = q == 0 ? (1 << B0) : (1 << B1);
      const uint16_t *src = (q == 0 ? d0.lut : d1.lut) + lut_index(strips[q], t, 0, 0, n_kt, nq) +
                            8 * std::min(i, 2 * nq - 1);
      lds_dma<16>(src, a + kTABytes + kTBBytes + wave * St::kMeta);
    } else {
      dma_codes<B0>(rc0, strips[0], t, n_kt, b);
      dma_codes<B1>(rc1, strips[1], t, n_kt, b + 1024);
      // lane l: strip q = (l / 16) % 2, row l % 16
      const int q = (lane >> 4) & 1;
      const BlockDesc &dq = q == 0 ? d0 : d1;
      const uint64_t mi = meta_index(q == 0 ? strips[0] : strips[1], t, lane & 15, 0, n_kt, GPT);
      uint8_t *m = a + kTABytes + kTBBytes + wave * St::kMeta;
      lds_dma<2 * GPT>(dq.scales + mi, m);       // dword slot per lane
      lds_dma<GPT>(dq.zeros + mi, m + 256);      // zero-extended dword slot per lane
    }
  }

  // the codes, scales and zeros of the wave's strips from the stage at sb
  __device__ __forceinline__ void load_codes(uint32_t sb, Tile0 &t0, Tile1 &t1) const {
    const int r = threadIdx.x & 15;
    const uint8_t *b = lds + sb + kTABytes + 2 * wave * 1024;
    const uint8_t *m = lds + sb + kTABytes + kTBBytes + wave * St::kMeta;
    if constexpr (PLANE) {
      lds_planes<B0>(b, t0);
      lds_planes<B1>(b + 1024, t1);
      lds_lut<B0>(m, t0);
      lds_lut<B1>(m + 512, t1);
    } else {
      lds_codes<B0>(b, t0);
      lds_codes<B1>(b + 1024, t1);
      const uint32_t *sc = reinterpret_cast<const uint32_t *>(m);
      const uint32_t *zz = reinterpret_cast<const uint32_t *>(m + 256);
      t0.sc = sc[r]; t1.sc = sc[16 + r];
      t0.zz = zz[r]; t1.zz = zz[16 + r];
    }
  }

  // activation fragments of step j of the tile in the stage at sb
  template <int NT>
  __device__ __forceinline__ void load_a(uint32_t sb, int j, f16x8 *av) const {
#pragma unroll
    for (int s = 0; s < NT; ++s) av[s] = tlds_a(lds + sb, s, j);
  }

  __device__ __forceinline__ static void decode(const Tile0 &t0, const Tile1 &t1, int j, f16x8 *w) {
    if constexpr (PLANE) {
      w[0] = plane_bop<B0>(t0.w, j, t0.L);
      w[1] = plane_bop<B1>(t1.w, j, t1.L);
    } else {
      w[0] = tdecode<B0, GPT>(t0, j);
      w[1] = tdecode<B1, GPT>(t1, j);
    }
  }

  // the two MFMAs of token sub-tile s of a step
  template <int NT>
  __device__ __forceinline__ static void mma_s(f16x8 av, const f16x8 *w, f32x4 (*acc)[NT], int s) {
    acc[0][s] = mfma16(av, w[0], acc[0][s]);
    acc[1][s] = mfma16(av, w[1], acc[1][s]);
  }

  // One 32-column step: the MFMAs of the step (weights wc, activation
  // fragments av), each fragment replaced by the next step's (step jn of
  // the stage at sn) once its MFMAs are issued, and the next step's
  // weights decoded into wn between them.
  template <int NT>
  __device__ __forceinline__ void step(f16x8 *av, const f16x8 *wc, f16x8 *wn, f32x4 (*acc)[NT], uint32_t sn,
                                       int jn, const Tile0 &t0, const Tile1 &t1) const {
    decode(t0, t1, jn, wn);
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      mma_s<NT>(av[s], wc, acc, s);
      av[s] = tlds_a(lds + sn, s, jn);
    }
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // The K walk as a software pipeline over 32-column steps: while the
  // MFMAs of step j run, the activation fragments of step j + 1 are read
  // and its weights decoded.  Tile t + 1's stage is opened (wait for its
  // transfers, barrier) before the last step of tile t, whose weights are
  // already decoded, so that step reads tile t + 1's codes and first
  // activation fragments and decodes its first step.  With N stages
  // transfers run N tiles ahead; tile t + N goes into tile t's stage once
  // every wave has passed that barrier with all its reads of the stage
  // completed.
  template <int NT>
  __device__ __forceinline__ void run(f32x4 (*acc)[NT]) const {
    constexpr int N = St::kN;
    issue(0, 0);
    issue(std::min(1, n_kt - 1), St::kBytes);
    if constexpr (N == 3) issue(std::min(2, n_kt - 1), 2 * St::kBytes);
    vm_wait<(N - 1) * kDma>();
    __builtin_amdgcn_s_barrier();
    Tile0 t0;
    Tile1 t1;
    f16x8 av[NT], w0[2], w1[2];
    load_codes(0, t0, t1);
    load_a<NT>(0, 0, av);
    decode(t0, t1, 0, w0);
    uint32_t sb = 0;     // stage of tile t
#pragma unroll 1
    for (int t = 0; t < n_kt; ++t) {
      step<NT>(av, w0, w1, acc, sb, 1, t0, t1);
      step<NT>(av, w1, w0, acc, sb, 2, t0, t1);
      step<NT>(av, w0, w1, acc, sb, 3, t0, t1);
      // open tile t + 1 (on the last tile: a stage of re-read data whose
      // values go unused)
      lgkm_vm_wait<(N - 2) * kDma>();
      __builtin_amdgcn_s_barrier();
      const uint32_t sn = sb == (N - 1) * St::kBytes ? 0u : sb + St::kBytes;
      issue(std::min(t + N, n_kt - 1), sb);
      load_codes(sn, t0, t1);
      __builtin_amdgcn_sched_barrier(0);
      step<NT>(av, w1, w0, acc, sn, 0, t0, t1);
      sb = sn;
    }
    // the queued re-reads of the last tile land before the LDS is reused
    vm_wait<0>();
    __syncthreads();
  }
};

// Workgroup b of n (n a multiple of 8): workgroups are dealt to the 8 XCDs
// round-robin, so logical tile L = (b % 8) * (n / 8) + b / 8 gives each
// XCD a contiguous run of tiles.
__device__ __forceinline__ int xcd_tile(int b, int n) { return (b & 7) * (n >> 3) + (b >> 3); }

// Buffer resource over a block's codes: the INT code region, or the top B
// bit-planes (stored top plane first, plane_bytes apart).
template <int B, bool PLANE>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t code_rsrc(const BlockDesc &d) {
  if constexpr (PLANE) return make_rsrc(d.codes, (uint32_t)B * (uint32_t)d.plane_bytes);
  else return make_rsrc(d.codes, code_region_bytes(d));
}

// gate/up: wave w owns I rows nt*128 + 16 w + [0, 16) of gate (q = 0) and
// up (q = 1), for all 128 tokens of the tile.
template <int BG, int BU, int GPT, bool PLANE>
__device__ __forceinline__ void tiled_gateup_body(const FfnArgs &a, const Chunk &ch, int nt, uint8_t *lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BlockDesc dg = a.desc[3 * ch.e], du = a.desc[3 * ch.e + 1];
  const int sg = nt * 8 + wave;
  const int strips[2] = {sg, sg};
  uint32_t rowoff[4];          // activation rows this lane moves: 16 w + 4 i + lane / 16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = std::min(16 * wave + 4 * i + (lane >> 4), ch.cnt - 1);
    rowoff[i] = (uint32_t)(a.sorted_pairs[ch.base + m] / a.k) * (uint32_t)a.H;
  }
  // the rows' x exponents: requested now, stored past the LDS stages after
  // the K walk (so that nothing waits for them)
  const int preg = threadIdx.x < kTM ? a.sorted_pairs[ch.base + std::min((int)threadIdx.x, ch.cnt - 1)] : 0;
  const int kreg = threadIdx.x < kTM ? a.xexp[preg / a.k] : 0;
  f32x4 acc[2][8];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[q][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  const TKLoop<BG, BU, GPT, PLANE> kl{dg,
                               du,
                               strips,
                               a.H / kTileK,
                               wave,
                               rowoff,
                               lds,
                               make_rsrc(a.xn, (uint32_t)a.T * (uint32_t)a.H * 2u),
                                      code_rsrc<BG, PLANE>(dg),
                                      code_rsrc<BU, PLANE>(du)};
  // the low-rank epilogue's inputs (z rows for up to 64 columns from one
  // partial, and the first U operands) are requested before the K walk, so
  // the epilogue does not wait for memory (z rows not with two groups per
  // tile, whose decode state leaves no registers for them)
  const int zw = 2 * a.RZ;
  const bool zpre = GPT == 1 && a.comp_on && a.ks_gu == 1 && zw <= 64 && a.rs == 0;
  ZPre<8, kTiledWaves, 4> zp;
  if (zpre) z_preload<8, kTiledWaves, 4>(a.zp_gu, zw, zw, ch, zp);
  f16x8 ub[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
    ub[q] = a.comp_on && a.r > 0 ? lowrank_bop(q ? du.U : dg.U, a.r, strips[q] * 16 + (lane & 15), 0)
                                 : pack_b(0, 0, 0, 0);
  kl.template run<8>(acc);
  // acc holds W x~ (x~ = x 2^K, the normalised rows), as do the z rows
  int *s_kx = reinterpret_cast<int *>(lds + TStages<PLANE>::kLds);
  int *s_p = s_kx + kTM;
  if (threadIdx.x < kTM) {
    s_kx[threadIdx.x] = kreg;
    s_p[threadIdx.x] = preg;
  }
  __syncthreads();
  uint16_t *l16 = reinterpret_cast<uint16_t *>(lds);
  if (a.comp_on) {
    uint16_t *zs = l16;
    if (zpre) z_store<8, kTiledWaves, 4>(a, ch, s_kx, zp, zw, zs);
    else z_prologue<8, kTiledWaves>(a, true, a.zp_gu, zw, a.ks_stride_gu, a.ks_gu, zw, ch, zs);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const BlockDesc &d = q ? du : dg;
      const int row = strips[q] * 16 + (lane & 15);
      if (a.r > 0) lowrank_epi<8>(d.U, a.r, a.Rp, row, zs + q * a.RZ, zw, acc[q], ub[q]);
      if (a.rs > 0) lowrank_epi<8>(d.Us, a.rs, a.Rsp, row, zs + q * a.RZ + a.Rp, zw, acc[q]);
    }
    __syncthreads();
  }
  // h = SiLU(gate) * up (gate and up back in x's units) in fp32 into LDS
  // [128 tokens][128 columns]
  float *h32 = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * s + 4 * (lane >> 4) + i;
      const int K = -s_kx[m];
      const float gv = __builtin_ldexpf(acc[0][s][i], K), uv = __builtin_ldexpf(acc[1][s][i], K);
      h32[m * kH32S + 16 * wave + (lane & 15)] = gv / (1.0f + __expf(-gv)) * uv;
    }
  }
  __syncthreads();
  // coalesced rows, 16 threads (one DPP row) per token: the row's largest
  // |h| gives eb, then h 2^(kNormTop - eb) as fp16; eb goes to hblk for both
  // 64-column halves of this 128-column block
  const int tid = threadIdx.x, c8 = 8 * (tid & 15);
  constexpr int kRowsPerPass = kTiledWaves * 64 / 16;
#pragma unroll
  for (int i = 0; i < kTM / kRowsPerPass; ++i) {
    const int r = (tid >> 4) + kRowsPerPass * i;
    const f32x4 v0 = *reinterpret_cast<const f32x4 *>(h32 + r * kH32S + c8);
    const f32x4 v1 = *reinterpret_cast<const f32x4 *>(h32 + r * kH32S + c8 + 4);
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fabsf(v0[j]), __builtin_fabsf(v1[j])));
    const int eb = h_block_exp(dpp_row_max(mx));
    if (r < ch.cnt) {
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        o[j] = as_u32(f16x2{(f16)__builtin_ldexpf(v0[2 * j], kNormTop - eb), (f16)__builtin_ldexpf(v0[2 * j + 1], kNormTop - eb)});
        o[2 + j] = as_u32(f16x2{(f16)__builtin_ldexpf(v1[2 * j], kNormTop - eb), (f16)__builtin_ldexpf(v1[2 * j + 1], kNormTop - eb)});
      }
      *reinterpret_cast<u32x4 *>(a.h + (int64_t)(ch.base + r) * a.I + nt * kTileK + c8) = o;
      if ((tid & 15) < 2) a.hblk[(int64_t)(ch.base + r) * a.hblk_stride + 2 * nt + (tid & 15)] = (int8_t)eb;
      if ((tid & 15) == 0) h_pair_exp(a, ch.base + r, s_p[r], eb);
    }
  }
}

// down: wave w owns H rows nt*256 + 32 w + [0, 32).
template <int BD, int GPT, bool PLANE>
__device__ __forceinline__ void tiled_down_body(const FfnArgs &a, const Chunk &ch, int nt, uint8_t *lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BlockDesc d = a.desc[3 * ch.e + 2];
  const int s0 = nt * 16 + 2 * wave;
  const int strips[2] = {s0, s0 + 1};
  uint32_t rowoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = std::min(16 * wave + 4 * i + (lane >> 4), ch.cnt - 1);
    rowoff[i] = (uint32_t)(ch.base + m) * (uint32_t)a.I;       // rows of the normalised h
  }
  f32x4 acc[2][8];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[q][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  const __amdgpu_buffer_rsrc_t rc = code_rsrc<BD, PLANE>(d);
  const TKLoop<BD, BD, GPT, PLANE> kl{d, d, strips, a.I / kTileK, wave, rowoff, lds,
                               make_rsrc(a.hn, (uint32_t)a.P * (uint32_t)a.I * 2u), rc, rc};
  kl.template run<8>(acc);
  if (a.comp_on) {
    uint16_t *zs = reinterpret_cast<uint16_t *>(lds);
    z_prologue<8, kTiledWaves>(a, false, a.zp_d, a.RZ, a.ks_stride_d, a.ks_d, a.RZ, ch, zs);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = strips[q] * 16 + (lane & 15);
      if (a.r > 0) lowrank_epi<8>(d.U, a.r, a.Rp, row, zs, a.RZ, acc[q]);
      if (a.rs > 0) lowrank_epi<8>(d.Us, a.rs, a.Rsp, row, zs + a.Rp, a.RZ, acc[q]);
    }
  }
  float *yp = a.ypart;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
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

// grid.x = (upper bound of token tiles) * (I / 128), rounded up to 8.
// PLANE: bit-plane blocks (GPT = 1, one LUT per 128-column tile), the
// committed q of each block in place of b.
template <int GPT, bool PLANE>
__global__ void __launch_bounds__(64 * kTiledWaves, 1) tiled_gateup_kernel(FfnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t tl_lds[];
  const int n_nt = a.I / kTileK;
  const int L = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = L / n_nt, nt = L % n_nt;
  Chunk ch;
  if (!find_chunk<kTM>(a.offsets, a.E, mt, &ch)) return;
  const int bg = a.desc[3 * ch.e].bits, bu = a.desc[3 * ch.e + 1].bits;
  switch (bg * 4 + bu) {
    case 2 * 4 + 2: tiled_gateup_body<2, 2, GPT, PLANE>(a, ch, nt, tl_lds); break;
    case 2 * 4 + 3: tiled_gateup_body<2, 3, GPT, PLANE>(a, ch, nt, tl_lds); break;
    case 2 * 4 + 4: tiled_gateup_body<2, 4, GPT, PLANE>(a, ch, nt, tl_lds); break;
    case 3 * 4 + 2: tiled_gateup_body<3, 2, GPT, PLANE>(a, ch, nt, tl_lds); break;
    case 3 * 4 + 3: tiled_gateup_body<3, 3, GPT, PLANE>(a, ch, nt, tl_lds); break;
    case 3 * 4 + 4: tiled_gateup_body<3, 4, GPT, PLANE>(a, ch, nt, tl_lds); break;
    case 4 * 4 + 2: tiled_gateup_body<4, 2, GPT, PLANE>(a, ch, nt, tl_lds); break;
    case 4 * 4 + 3: tiled_gateup_body<4, 3, GPT, PLANE>(a, ch, nt, tl_lds); break;
    default: tiled_gateup_body<4, 4, GPT, PLANE>(a, ch, nt, tl_lds); break;
  }
}

// grid.x = (upper bound of token tiles) * (H / 256), rounded up to 8
template <int GPT, bool PLANE>
__global__ void __launch_bounds__(64 * kTiledWaves, 1) tiled_down_kernel(FfnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t tl_lds[];
  const int n_nt = a.H / 256;
  const int L = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = L / n_nt, nt = L % n_nt;
  Chunk ch;
  if (!find_chunk<kTM>(a.offsets, a.E, mt, &ch)) return;
  switch (a.desc[3 * ch.e + 2].bits) {
    case 2: tiled_down_body<2, GPT, PLANE>(a, ch, nt, tl_lds); break;
    case 3: tiled_down_body<3, GPT, PLANE>(a, ch, nt, tl_lds); break;
    default: tiled_down_body<4, GPT, PLANE>(a, ch, nt, tl_lds); break;
  }
}

}  // namespace moeq
