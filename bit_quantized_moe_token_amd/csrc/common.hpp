// Shared device/host definitions of libmoeq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moeq.h"

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace moeq {

// --------------------------------------------------------------- layout --
// Weights of one block (N x K) are stored in strips of 16 rows and tiles of
// 128 columns.  A 16 x 128 tile is read by one wave: lane l owns row
// n = l % 16 and the columns 32*j + 8*(l/16) + i (j = 0..3, i = 0..7), which
// is the B-operand layout of v_mfma_f32_16x16x32_f16 for four consecutive
// 32-column steps j.  Tiles are grouped by four so that each lane reads its
// data for four tiles with 128-bit loads.
constexpr int kStripRows = 16;
constexpr int kTileK = 128;
constexpr int kTilesPerGroup = 4;
constexpr int kWave = 64;

// Per-block record in device memory, written by moeq_pack.
struct BlockDesc {
  const uint8_t *codes;   // INT codes, or bit-plane 3 (MSB) of 4 planes
  uint64_t plane_bytes;   // bytes of one bit-plane region (bit-plane form)
  const uint16_t *scales; // tiled fp16 scales (INT)
  const uint8_t *zeros;   // tiled zeros (INT)
  const uint16_t *lut;    // tiled LUT, 2^q fp16 per (row, tile) (bit-plane)
  const uint16_t *U;      // per-expert U [N, r] (nullptr when r == 0)
  const uint16_t *V;      // per-expert V [r, K]
  const uint16_t *Us;     // shared U of this expert's group [N, rs] or nullptr
  const uint16_t *Vs;     // shared V [rs, K]
  int32_t N, K, bits, fmt;
};

struct LayerDims {
  int32_t E, H, I, G, fmt, r, rs, share;
};

// Host-side error reporting (thread local).
void set_error(const char *fmt, ...);
moeq_status fail(moeq_status s, const char *fmt, ...);
moeq_status check_launch(const char *what);

// Profiling hooks around launches (no-ops unless enabled).
void prof_begin(const char *name, hipStream_t s);
void prof_end(const char *name, hipStream_t s);

// ------------------------------------------------------ device helpers --

// Loads through the global address space (the pointers handed to kernels
// are generic; telling the compiler lets it use global_load and the vector
// memory counter only).
template <typename T>
__device__ __forceinline__ T gld(const void *p) {
  return *(const __attribute__((address_space(1))) T *)(p);
}

// Non-temporal global load: for data read once per call (packed weights),
// so that it streams past the caches instead of displacing reused data.
template <typename T>
__device__ __forceinline__ T gld_nt(const void *p) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) T *)(p));
}

// (a & m) | c as one v_and_or_b32.  A VOP3 instruction on this target
// takes no literal operand, so with literal m and c the compiler would emit
// a v_and_b32 and a v_or_b32; the asm operands make it keep the constants
// in registers (hoisted out of loops) and issue the single instruction.
// Its result must not be an MFMA operand without a compiler-emitted
// instruction in between: the compiler does not count inline asm when it
// inserts the wait states between a VALU write and an MFMA read.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

__device__ __forceinline__ f16x2 as_h2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Global -> LDS transfer of SIZE bytes per lane (global_load_lds): the
// compiler does not track these LDS writes, so callers wait with vm_wait
// before reading the data and order LDS reuse themselves.
template <int SIZE>
__device__ __forceinline__ void lds_dma(const void *src, uint8_t *lds_base) {
  const auto g = (const __attribute__((address_space(1))) void *)src;
  const auto l = (__attribute__((address_space(3))) void *)lds_base;
  if constexpr (SIZE == 16) __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
  else if constexpr (SIZE == 4) __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
  else if constexpr (SIZE == 2) __builtin_amdgcn_global_load_lds(g, l, 2, 0, 0);
  else __builtin_amdgcn_global_load_lds(g, l, 1, 0, 0);
}

// Note on the LDS layout of these transfers: lane l's bytes land at
// base + l * size for 16- and 4-byte transfers; 1- and 2-byte transfers
// fill a zero-extended dword slot at base + 4 l.

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt left at
// their maxima).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The same with every LDS read (and scalar load) of this wave completed too
// (lgkmcnt 0).
template <int N>
__device__ __forceinline__ void lgkm_vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Buffer resource over [base, base + bytes) for the raw buffer loads below
// (dword 3: the gfx9 default data format; offsets past `bytes` read zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Buffer -> LDS transfer of SIZE (4 or 16) bytes per lane from
// base + soff + voff (voff per lane, soff uniform): lane l's bytes land at
// lds_base + l * SIZE.  Like lds_dma, untracked by the compiler.
template <int SIZE>
__device__ __forceinline__ void lds_dma_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t *lds_base) {
  const auto l = (__attribute__((address_space(3))) void *)lds_base;
  if constexpr (SIZE == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff, soff, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 4, voff, soff, 0, 0);
}

__device__ __forceinline__ f16x8 pack_b(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(f16x8, v);
}

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---- power-of-two normalisation of fp16 activations.  Activations (x)
// and the SwiGLU output (h) are held in fp16 scaled by an exact power of
// two so that their largest magnitude per token (per pair for h) lies in
// [2^kNormTop, 2^(kNormTop+1)): their relative precision then does not
// depend on their absolute size.  The scale is undone in fp32.
constexpr int kNormTop = 6;
constexpr int kNoExp = -1000;   // exponent of an all-zero row or block

// floor(log2 |v|) of a finite float (denormals included); kNoExp for 0.
__device__ __forceinline__ int ilogb_f32(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v) & 0x7fffffffu;
  if (b == 0) return kNoExp;
  const int e = (int)(b >> 23);
  return e ? e - 127 : (31 - __builtin_clz(b)) - 149;
}

// floor(log2 m) of an fp16 magnitude given by its bits (sign cleared).
__device__ __forceinline__ int ilogb_f16bits(uint32_t m) {
  if (m == 0) return kNoExp;
  const int e = (int)(m >> 10);
  return e ? e - 15 : (31 - __builtin_clz(m)) - 24;
}

// Exponent K of x~ = x * 2^K for a token whose largest |x| has
// floor(log2) = e: the largest lands in [2^kNormTop, 2^(kNormTop+1)).  K is
// capped at 15 so that 2^K stays an fp16 number (rows whose largest value
// is below 2^(kNormTop-15) are scaled by 2^15 and stay smaller).
__device__ __forceinline__ int x_norm_exp(int e) { return e >= kNormTop - 15 ? kNormTop - e : 15; }

// fp16 bits of 2^e for e <= 15 (subnormal from -15 down to -24; 0 below).
__host__ __device__ constexpr uint32_t f16_pow2_bits(int e) {
  return e < -24 ? 0u : e < -14 ? (1u << (e + 24)) : (uint32_t)(e + 15) << 10;
}

// (2^e, 2^e) as an fp16 pair, e <= 15 (0 below 2^-24): the fp32 power of
// two converted once (exact; 2^-25 and below round to 0).
__device__ __forceinline__ uint32_t f16x2_pow2(int e) {
  const f16 h = (f16)__builtin_ldexpf(1.0f, e);
  return as_u32(f16x2{h, h});
}

// Multiply the eight fp16 values of v by the fp16 pair m (exact for powers
// of two unless the result is subnormal).
// (The elements go through as_h2 by value: a bit_cast applied directly to
// a vector-element expression v[i] reads element 0 with this compiler.)
__device__ __forceinline__ u32x4 scale_f16x8(u32x4 v, uint32_t m) {
  const f16x2 mm = as_h2(m);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = as_u32(as_h2(v[i]) * mm);
  return r;
}

// Largest value over the 16 lanes of each DPP row (quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror, row_mirror).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, true);
}
__device__ __forceinline__ float dpp_row_max(float v) {
  v = __builtin_fmaxf(v, __builtin_bit_cast(float, dpp_i<0xb1>(__builtin_bit_cast(int, v))));
  v = __builtin_fmaxf(v, __builtin_bit_cast(float, dpp_i<0x4e>(__builtin_bit_cast(int, v))));
  v = __builtin_fmaxf(v, __builtin_bit_cast(float, dpp_i<0x141>(__builtin_bit_cast(int, v))));
  return __builtin_fmaxf(v, __builtin_bit_cast(float, dpp_i<0x140>(__builtin_bit_cast(int, v))));
}
__device__ __forceinline__ float dpp_half_row_max(float v) {   // over the 8 lanes of each half-row
  v = __builtin_fmaxf(v, __builtin_bit_cast(float, dpp_i<0xb1>(__builtin_bit_cast(int, v))));
  v = __builtin_fmaxf(v, __builtin_bit_cast(float, dpp_i<0x4e>(__builtin_bit_cast(int, v))));
  return __builtin_fmaxf(v, __builtin_bit_cast(float, dpp_i<0x141>(__builtin_bit_cast(int, v))));
}
__device__ __forceinline__ int dpp_row_max(int v) {
  v = __builtin_elementwise_max(v, dpp_i<0xb1>(v));
  v = __builtin_elementwise_max(v, dpp_i<0x4e>(v));
  v = __builtin_elementwise_max(v, dpp_i<0x141>(v));
  return __builtin_elementwise_max(v, dpp_i<0x140>(v));
}

// Round a float64 to the nearest fp16 (ties to even), directly from the
// double's bits so there is exactly one rounding.  Finite inputs only.
__host__ __device__ inline uint16_t f64_to_f16_bits(double d) {
  uint64_t b;
  __builtin_memcpy(&b, &d, 8);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  int exp = (int)((b >> 52) & 0x7ff);
  uint64_t mant = b & ((1ull << 52) - 1);
  if (exp == 0) return sign;                      // zero or double subnormal
  int e = exp - 1023;                             // unbiased
  if (e > 15) return sign | 0x7c00u;              // overflow -> inf
  uint64_t sig = mant | (1ull << 52);             // 53-bit significand
  int shift;                                      // bits to drop
  uint32_t hexp;
  if (e >= -14) {                                 // normal fp16
    shift = 42;
    hexp = (uint32_t)(e + 15);
  } else {                                        // subnormal fp16
    shift = 42 + (-14 - e);
    hexp = 0;
    if (shift > 53 + 1) return sign;              // rounds to zero
  }
  uint64_t q = sig >> shift;
  uint64_t rem = sig & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) q += 1;
  uint32_t out;
  if (hexp == 0) {
    out = (uint32_t)q;                            // may carry into exponent 1
  } else {
    // q holds the implicit bit at position 10; carry may bump the exponent
    out = (hexp << 10) + (uint32_t)(q - (1u << 10));
    if (q >= (1u << 11)) out = ((hexp + 1) << 10);
  }
  if (out >= 0x7c00u) out = 0x7c00u;
  return sign | (uint16_t)out;
}

__host__ __device__ inline double f16_bits_to_f64(uint16_t h) {
  uint32_t sign = h >> 15, exp = (h >> 10) & 0x1f, mant = h & 0x3ff;
  double v;
  if (exp == 0) v = (double)mant * (1.0 / 16777216.0);               // 2^-24
  else if (exp == 31) v = mant ? __builtin_nan("") : __builtin_inf();
  else v = (double)(mant | 0x400) * __builtin_ldexp(1.0, (int)exp - 25);
  return sign ? -v : v;
}

}  // namespace moeq

#define MOEQ_API extern "C" __attribute__((visibility("default")))
