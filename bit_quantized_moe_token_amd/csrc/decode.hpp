// In-register decode of packed low-bit weights into fp16 MFMA operands.
//
// A lane holds 32 codes of one row per 16 x 128 tile: pair P = 4*j + v is
// the two codes at columns 32*j + 8*(l/16) + 2*v (+1), i.e. register v of
// the 16x16x32 MFMA B operand of step j.
//
// INT packing (4*b bytes per lane per tile).  Every pair is one "field":
// its two codes sit at bits [p, p+b) of the low and the high half of
// (d[e] >> s), so one shift (shared by the fields of a dword) and one AND
// give both codes of the pair as fp16 bit fields at offset p.  The offset p
// depends only on v (the same for all four MFMA steps of a tile):
//   b = 4: p = (0, 4, 0, 4); dword j holds step j, pair v at bits 4v / 16+4v.
//   b = 2: p = (0, 2, 4, 6); dword e holds pairs 8e..8e+7 at bits 2u / 16+2u
//          (u = P % 8; u >= 4 read from d >> 8).
//   b = 3: p = (0, 1, 4, 7); each half-dword holds five 3-bit fields and one
//          spare bit (d0, d1: spare bit 0, fields at 1, 4, 7, 10, 13;
//          d2: spare bit 6, fields at 0, 3, 7, 10, 13).  The spare bits of
//          d0, d1, d2 form the three bits of pair 12; the other 15 pairs
//          are listed in int_field<3>.
// Two decodes are built on the fields:
//   - exact-integer ("magic") form: OR-ing a field into the mantissa of
//     1024.0 (0x6400) gives 1024 + c 2^p; one packed FMA turns it into
//     (c - z) exactly (tiled kernels, read-back);
//   - subnormal form: the AND alone, read as fp16, is the subnormal number
//     c 2^(p - 24).  Multiplied by activations pre-scaled by 2^-p per column
//     it gives c x 2^-24 exactly inside the MFMA (streaming kernels).
// Bit-plane packing (4 bytes per plane per lane per tile): the bit of code
// plane c for register element i = 2v + h of step j (pair P = 4j + v, half
// h) is at bit 8 (i mod 4) + 4 (i div 4) + j, rotated left by c.  The four
// weights of a quad (elements 4qd .. 4qd + 3 of a step) thus sit at bit
// s + c of the four bytes (s = 4qd + j), so a mask per plane and one
// rotation of their OR put a quad's indices one per byte, plane c at bit c
// (then down by 4 - q): the byte selectors of v_perm.
#pragma once
#include "common.hpp"

namespace moeq {

constexpr uint32_t kMagic = 0x64006400u;   // (1024.0, 1024.0) in fp16

struct Field {
  int e, s, p;   // dword, right shift, bit offset of the field after the shift
};

// Field of pair P of a b-bit INT tile (e < 0: the spare-bit pair of b = 3).
template <int B>
__host__ __device__ constexpr Field int_field(int P) {
  if (B == 4) return Field{P >> 2, (P & 3) >= 2 ? 8 : 0, (P & 1) ? 4 : 0};
  if (B == 2) return Field{P >> 3, (P & 7) >= 4 ? 8 : 0, 2 * (P & 3)};
  switch (P) {
    case 0: return Field{2, 0, 0};
    case 1: return Field{0, 0, 1};
    case 2: return Field{0, 0, 4};
    case 3: return Field{0, 6, 7};
    case 4: return Field{2, 3, 0};
    case 5: return Field{0, 6, 1};
    case 6: return Field{0, 6, 4};
    case 7: return Field{1, 6, 7};
    case 8: return Field{2, 13, 0};
    case 9: return Field{1, 0, 1};
    case 10: return Field{1, 0, 4};
    case 11: return Field{2, 0, 7};
    case 12: return Field{-1, 0, 0};
    case 13: return Field{1, 6, 1};
    case 14: return Field{1, 6, 4};
    default: return Field{2, 3, 7};
  }
}

// Field offset of register v of every step (the column pattern).
template <int B>
__host__ __device__ constexpr int int_pattern(int v) {
  return int_field<B>(v).p;
}

// Spare-bit position of the b = 3 pair 12: bit i of both codes is bit
// spare3_bit(i) (+16) of dword i.
__host__ __device__ constexpr int spare3_bit(int i) { return i == 2 ? 6 : 0; }

// Both fields of pair P at offset p of each half (no bias).
template <int B>
__device__ __forceinline__ uint32_t int_pair_bits(const uint32_t *d, int P) {
  constexpr uint32_t kOne = 0x00010001u;
  // Plain operations only: this value feeds an MFMA operand directly, and
  // the compiler inserts the wait states such a read needs only after
  // instructions it emitted itself (not after inline asm).
  if constexpr (B == 3) {
    if (P == 12) return (d[0] & kOne) | ((d[1] << 1) & 2 * kOne) | ((d[2] >> 4) & 4 * kOne);
  }
  const Field f = int_field<B>(P);
  return (d[f.e] >> f.s) & (((1u << B) - 1) << f.p) * kOne;
}

// Biased pair: 1024 + c 2^p in each fp16 half.
template <int B>
__device__ __forceinline__ uint32_t int_pair_raw(const uint32_t *d, int P) {
  constexpr uint32_t kOne = 0x00010001u;
  if constexpr (B == 3) {
    if (P == 12) {
      uint32_t m = and_or(d[0], kOne, kMagic);
      m = and_or(d[1] << 1, 2 * kOne, m);
      return and_or(d[2] >> 4, 4 * kOne, m);
    }
  }
  const Field f = int_field<B>(P);
  return and_or(d[f.e] >> f.s, (((1u << B) - 1) << f.p) * kOne, kMagic);
}

template <int B>
__device__ __forceinline__ constexpr int int_pair_shift(int P) {
  return int_pattern<B>(P & 3);
}

// Per-(row, group) constants turning a biased pair into (c - z) exactly:
// (1024 + c 2^p) * 2^-p - (1024 * 2^-p + z) = c - z.  The fp16 constant
// -(2^(10-p) + z) is built from the integer zero directly: exponent field
// 25 - p and mantissa z * 2^p (exact while z * 2^p < 1024, which holds for
// every field offset used: z < 2^b, p <= 10 - b).  With the zero
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
  const uint16_t b = (uint16_t)((15 - p) << 10);
  const f16 m = __builtin_bit_cast(f16, b);
  return f16x2{m, m};
}

__device__ __forceinline__ f16x2 pk_fma(f16x2 a, f16x2 b, f16x2 c) {
  return __builtin_elementwise_fma(a, b, c);
}

// Pair constants for the field offsets of a b-bit tile (indexed by p; the
// other slots are left untouched); z is the integer zero of the group.
template <int B>
__device__ __forceinline__ void fill_pair_consts(PairConst *pc, uint32_t z) {
  const uint32_t z2 = z | (z << 16);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int p = int_pattern<B>(v);
    pc[p].add = (z2 << p) | pair_add_base(p);
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

// Subnormal-form B operand of step j: register v holds c 2^(p_v - 24) for
// both codes of pair 4j + v.
template <int B>
__device__ __forceinline__ f16x8 int_bop_sub(const uint32_t *d, int j) {
  return pack_b(int_pair_bits<B>(d, 4 * j + 0), int_pair_bits<B>(d, 4 * j + 1),
                int_pair_bits<B>(d, 4 * j + 2), int_pair_bits<B>(d, 4 * j + 3));
}

// Constant B operand -2^(p_v - 24) (subnormal): against activations
// pre-scaled by 2^-p_v it sums -2^-24 x over the step's 32 columns, the
// same value in every output column.
template <int B>
__device__ __forceinline__ f16x8 int_bop_sum() {
  return pack_b((0x8000u | (1u << int_pattern<B>(0))) * 0x10001u, (0x8000u | (1u << int_pattern<B>(1))) * 0x10001u,
                (0x8000u | (1u << int_pattern<B>(2))) * 0x10001u, (0x8000u | (1u << int_pattern<B>(3))) * 0x10001u);
}

// Pre-scale of the activations of register v of an A operand (or of the
// same columns in a staged row): multiply by 2^-p_v.
template <int B>
__device__ __forceinline__ uint32_t prescale_pair(uint32_t x, int v) {
  return as_u32(as_h2(x) * pair_mul(int_pattern<B>(v)));
}

// Re-scale an A operand pre-scaled for b0 to the pattern of b1.
template <int B0, int B1>
__device__ __forceinline__ f16x8 rescale_a(f16x8 a) {
  if constexpr (B0 == B1) {
    return a;
  } else {
    const u32x4 w = __builtin_bit_cast(u32x4, a);
    u32x4 r;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int d = int_pattern<B0>(v) - int_pattern<B1>(v);
      const uint16_t b = (uint16_t)((15 + d) << 10);
      const f16 m = __builtin_bit_cast(f16, b);
      r[v] = d == 0 ? w[v] : as_u32(as_h2(w[v]) * f16x2{m, m});
    }
    return __builtin_bit_cast(f16x8, r);
  }
}

// Bit of element i (0..7) of step j in a plane dword.
__host__ __device__ constexpr int plane_bit(int j, int i) { return 8 * (i % 4) + 4 * (i / 4) + j; }

// The low min(q, 3) bits of the q-bit indices of a quad, weight e in byte
// e, from the top q planes (pl[u] = plane 3 - u; plane c is index bit
// c - (4 - q)); s = 4 qd + j.
template <int Q>
__device__ __forceinline__ uint32_t plane_sel(const uint32_t *pl, int s) {
  uint32_t t = 0;
#pragma unroll
  for (int u = Q > 3 ? 1 : 0; u < Q; ++u) t |= pl[u] & __builtin_rotateleft32(0x01010101u, s + 3 - u);
  return __builtin_rotateright32(t, s + 4 - Q);
}

// q = 4: selector that takes byte e from the entries-8..15 lookup when
// index bit 3 of weight e (plane 3) is set, else from the entries-0..7
// lookup.
__device__ __forceinline__ uint32_t plane_top(const uint32_t *pl, int s) {
  return __builtin_rotateright32(pl[0] & __builtin_rotateleft32(0x01010101u, s + 3), s + 1) | 0x03020100u;
}

// Full q-bit index of weight e of a quad (debug read-back).
template <int Q>
__device__ __forceinline__ uint32_t plane_index(const uint32_t *pl, int s, int e) {
  const uint32_t lo = (plane_sel<Q>(pl, s) >> (8 * e)) & 7u;
  if constexpr (Q < 4) return lo;
  else return lo | (((plane_top(pl, s) >> (8 * e + 2)) & 1u) << 3);
}

// One byte (low or high) of the LUT entries of a quad's four weights from
// that byte's table T (2^q bytes in 2^q / 4 dwords, entry i in byte i).
template <int Q>
__device__ __forceinline__ uint32_t quad_bytes(const uint32_t *T, uint32_t sel, uint32_t top) {
  if constexpr (Q == 2) return __builtin_amdgcn_perm(T[0], T[0], sel);
  else if constexpr (Q == 3) return __builtin_amdgcn_perm(T[1], T[0], sel);
  else return __builtin_amdgcn_perm(__builtin_amdgcn_perm(T[3], T[2], sel), __builtin_amdgcn_perm(T[1], T[0], sel), top);
}

// The quad's four fp16 weights as two dwords (elements 4qd, 4qd+1 and
// 4qd+2, 4qd+3) from the lane's row table L: the low bytes of the 2^q
// entries in 2^q / 4 dwords, then their high bytes.
template <int Q>
__device__ __forceinline__ void plane_quad(const uint32_t *pl, int s, const uint32_t *L, uint32_t &d0, uint32_t &d1) {
  const uint32_t sel = plane_sel<Q>(pl, s);
  const uint32_t top = Q == 4 ? plane_top(pl, s) : 0u;
  const uint32_t lo = quad_bytes<Q>(L, sel, top);
  const uint32_t hi = quad_bytes<Q>(L + (1 << Q) / 4, sel, top);
  d0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  d1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

}  // namespace moeq
