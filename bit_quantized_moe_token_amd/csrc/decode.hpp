// In-register decode of packed low-bit weights into fp16 MFMA operands.
//
// A lane holds 32 codes of one row per 16 x 128 tile: pair P = 4*j + v is
// the two codes at columns 32*j + 8*(l/16) + 2*v (+1), i.e. register v of
// the 16x16x32 MFMA B operand of step j.  Codes are pulled into fp16 lanes
// with one v_and_or_b32 per pair: OR-ing a code field into the mantissa of
// 1024.0 (0x6400) gives 1024 + c * 2^p where p is the field's bit offset.
// One packed FMA then removes the bias and the offset scale exactly.
//
// INT packing (4*b bytes per lane per tile):
//   b = 4: dword j holds step j; pair v: low code at bit 4v, high at 16+4v.
//   b = 3: dword e holds pairs 5e..5e+4 at bits 3u / 16+3u (u = 0..4);
//          pair 15 is spread over bits 15 (low) and 31 (high) of the three
//          dwords, bit e of each code in dword e.
//   b = 2: dword e holds pairs 8e..8e+7 at bits 2u / 16+2u.
// Bit-plane packing (4 bytes per plane per lane per tile): the bit of code
// plane c for the weight (pair P = 4j + v, half h) is at bit 16h + 4v + j.
#pragma once
#include "common.hpp"

namespace moeq {

constexpr uint32_t kMagic = 0x64006400u;   // (1024.0, 1024.0) in fp16

// Raw biased pair P of an INT tile and log2 of its field scale.
template <int B>
__device__ __forceinline__ uint32_t int_pair_raw(const uint32_t *d, int P);

template <>
__device__ __forceinline__ uint32_t int_pair_raw<4>(const uint32_t *d, int P) {
  const int j = P >> 2, v = P & 3;
  const uint32_t w = (v >= 2) ? (d[j] >> 8) : d[j];
  return and_or(w, (v & 1) ? 0x00F000F0u : 0x000F000Fu, kMagic);
}
template <>
__device__ __forceinline__ uint32_t int_pair_raw<3>(const uint32_t *d, int P) {
  if (P == 15) {
    uint32_t m = and_or(d[0] >> 15, 0x00010001u, kMagic);
    m = and_or(d[1] >> 14, 0x00020002u, m);
    return and_or(d[2] >> 13, 0x00040004u, m);
  }
  const int e = P / 5, u = P % 5;
  const uint32_t w = (u >= 3) ? (d[e] >> 9) : d[e];
  const int uu = (u >= 3) ? u - 3 : u;
  return and_or(w, 0x00070007u << (3 * uu), kMagic);
}
template <>
__device__ __forceinline__ uint32_t int_pair_raw<2>(const uint32_t *d, int P) {
  const int e = P >> 3, u = P & 7;
  const uint32_t w = (u >= 5) ? (d[e] >> 10) : d[e];
  const int uu = (u >= 5) ? u - 5 : u;
  return and_or(w, 0x00030003u << (2 * uu), kMagic);
}

// log2 of the field scale of pair P (constant-folded when P is).
template <int B>
__device__ __forceinline__ constexpr int int_pair_shift(int P) {
  if (B == 4) return ((P & 3) & 1) ? 4 : 0;
  if (B == 3) {
    if (P == 15) return 0;
    const int u = P % 5;
    return 3 * ((u >= 3) ? u - 3 : u);
  }
  const int u = P & 7;
  return 2 * ((u >= 5) ? u - 5 : u);
}

// Per-(row, group) constants turning a biased pair into (c - z) exactly:
// (1024 + c 2^p) * 2^-p - (1024 * 2^-p + z) = c - z.  The fp16 constant
// -(2^(10-p) + z) is built from the integer zero directly: exponent field
// 25 - p and mantissa z * 2^p (exact while z * 2^p < 1024, which holds for
// every field of the b-bit layouts: z < 2^b, p <= 10 - b).  With the zero
// duplicated into both halves once per group, each constant is one
// shift-or.
struct PairConst {
  uint32_t add;   // fp16 pair -(2^(10-p) + z)
};

__device__ __forceinline__ constexpr uint32_t pair_add_base(int p) {
  return (0x8000u | ((uint32_t)(25 - p) << 10)) * 0x10001u;
}

// 2^-p as an fp16 pair (p is a constant after unrolling).
__device__ __forceinline__ f16x2 pair_mul(int p) {
  const f16 m = (f16)(p == 2 ? 0.25f : p == 3 ? 0.125f : p == 4 ? 0.0625f : p == 6 ? 0.015625f
                      : p == 8 ? 0.00390625f : 1.0f);
  return f16x2{m, m};
}

__device__ __forceinline__ f16x2 pk_fma(f16x2 a, f16x2 b, f16x2 c) {
  return __builtin_elementwise_fma(a, b, c);
}

// Pair constants for every field scale a b-bit tile uses (indexed by the
// field's bit offset p; unused slots are left untouched); z is the integer
// zero of the group.
template <int B>
__device__ __forceinline__ void fill_pair_consts(PairConst *pc, uint32_t z) {
  const uint32_t z2 = z | (z << 16);
  if (B == 4) { pc[0].add = z2 | pair_add_base(0); pc[4].add = (z2 << 4) | pair_add_base(4); }
  if (B == 3) {
    pc[0].add = z2 | pair_add_base(0); pc[3].add = (z2 << 3) | pair_add_base(3);
    pc[6].add = (z2 << 6) | pair_add_base(6);
  }
  if (B == 2) {
    pc[0].add = z2 | pair_add_base(0); pc[2].add = (z2 << 2) | pair_add_base(2);
    pc[4].add = (z2 << 4) | pair_add_base(4); pc[6].add = (z2 << 6) | pair_add_base(6);
    pc[8].add = (z2 << 8) | pair_add_base(8);
  }
}

// (c - z) for both codes of pair P as an fp16 pair (exact small integers);
// pc holds the constants of fill_pair_consts<B>.
template <int B>
__device__ __forceinline__ uint32_t int_pair_cz(const uint32_t *d, int P, const PairConst *pc) {
  const uint32_t raw = int_pair_raw<B>(d, P);
  const int p = int_pair_shift<B>(P);
  if (p == 0) return as_u32(as_h2(raw) + as_h2(pc[0].add));
  return as_u32(pk_fma(as_h2(raw), pair_mul(p), as_h2(pc[p].add)));
}

// Merged q-bit indices of MFMA step j from the top q planes (pl[0] = plane
// 3): nibble v of the low half is the index of the low weight of pair v,
// nibble v of the high half that of the high weight.
template <int Q>
__device__ __forceinline__ uint32_t plane_merge(const uint32_t *pl, int j) {
  uint32_t m = 0;
#pragma unroll
  for (int u = 0; u < Q; ++u) m |= ((pl[u] >> j) & 0x11111111u) << (Q - 1 - u);
  return m;
}

// LUT lookup of a pair of q-bit indices w = i_lo | i_hi << 16 in the lane's
// row table L (2^q fp16 entries in 2^(q-1) dwords).
template <int Q>
__device__ __forceinline__ uint32_t lut_pair(uint32_t w, const uint32_t *L) {
  const uint32_t sel = (w & 0x00030003u) * 0x0202u + 0x01000100u;
  if (Q == 2) return __builtin_amdgcn_perm(L[1], L[0], sel);
  const uint32_t r0 = __builtin_amdgcn_perm(L[1], L[0], sel);
  const uint32_t r1 = __builtin_amdgcn_perm(L[3], L[2], sel);
  const uint32_t m2 = ((w >> 2) & 0x00010001u) * 0xFFFFu;
  const uint32_t a = (m2 & r1) | (~m2 & r0);
  if (Q == 3) return a;
  const uint32_t r2 = __builtin_amdgcn_perm(L[5], L[4], sel);
  const uint32_t r3 = __builtin_amdgcn_perm(L[7], L[6], sel);
  const uint32_t b = (m2 & r3) | (~m2 & r2);
  const uint32_t m3 = ((w >> 3) & 0x00010001u) * 0xFFFFu;
  return (m3 & b) | (~m3 & a);
}

}  // namespace moeq
