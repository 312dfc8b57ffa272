// Encoding of expert weights: asymmetric RTN group quantization and the
// bit-plane lookup tables (MiLo abstract: under-4-bit MoE quantization;
// PagedWeight review, Figure 3 caption: bit-plane format with a LUT of
// bitwidth-specific centroid values).  Offline work; float64 arithmetic so
// that every stored value is rounded exactly once.
#include "common.hpp"

namespace moeq {

// One thread per (row, group): scan the group's fp16 values for the range,
// round the scale to fp16 once, then emit codes.  Groups are independent.
__global__ void __launch_bounds__(256)
quantize_rtn_kernel(const uint16_t *__restrict__ w, int32_t N, int32_t K, int32_t G,
                    int32_t bits, uint8_t *__restrict__ codes, uint16_t *__restrict__ scales,
                    uint8_t *__restrict__ zeros) {
  const int64_t ng = K / G;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)N * ng) return;
  const int64_t n = gid / ng, g = gid % ng;
  const uint16_t *src = w + n * (int64_t)K + g * G;
  double lo = 0.0, hi = 0.0;
  for (int i = 0; i < G; ++i) {
    double v = f16_bits_to_f64(src[i]);
    lo = v < lo ? v : lo;
    hi = v > hi ? v : hi;
  }
  const double qmax = (double)((1 << bits) - 1);
  uint16_t s16 = f64_to_f16_bits((hi - lo) / qmax);
  if (hi == lo || (s16 & 0x7fffu) == 0) s16 = 0x3c00u;   // 1.0
  const double s = f16_bits_to_f64(s16);
  double z = rint(-lo / s);
  z = z < 0.0 ? 0.0 : (z > qmax ? qmax : z);
  uint8_t *dst = codes + n * (int64_t)K + g * G;
  for (int i = 0; i < G; ++i) {
    double c = rint(f16_bits_to_f64(src[i]) / s) + z;
    c = c < 0.0 ? 0.0 : (c > qmax ? qmax : c);
    dst[i] = (uint8_t)c;
  }
  scales[gid] = s16;
  zeros[gid] = (uint8_t)z;
}

// One thread per (row, group): bucket sums of the fp16 weights by q-bit
// index (exact in float64), then fp16(mean) or the bucket's mid-code value.
__global__ void __launch_bounds__(256)
build_lut_kernel(const uint16_t *__restrict__ w, const uint8_t *__restrict__ codes4,
                 const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
                 int32_t N, int32_t K, int32_t G, int32_t q, uint16_t *__restrict__ lut) {
  const int64_t ng = K / G;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)N * ng) return;
  const int64_t n = gid / ng, g = gid % ng;
  const uint16_t *src = w + n * (int64_t)K + g * G;
  const uint8_t *cs = codes4 + n * (int64_t)K + g * G;
  double sum[16];
  int cnt[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) { sum[j] = 0.0; cnt[j] = 0; }
  const int shift = 4 - q;
  for (int i = 0; i < G; ++i) {
    const int idx = (cs[i] & 15) >> shift;
    const double v = f16_bits_to_f64(src[i]);
#pragma unroll
    for (int j = 0; j < 16; ++j) {      // register-resident buckets
      if (j == idx) { sum[j] += v; cnt[j] += 1; }
    }
  }
  const double s = f16_bits_to_f64(scales[gid]);
  const double z = (double)zeros[gid];
  const int span = 1 << shift;
  uint16_t *out = lut + gid * 16;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint16_t v = 0;
    if (j < (1 << q)) {
      if (cnt[j] > 0) v = f64_to_f16_bits(sum[j] / (double)cnt[j]);
      else v = f64_to_f16_bits(s * ((double)(j * span) + 0.5 * (double)(span - 1) - z));
    }
    out[j] = v;
  }
}

}  // namespace moeq

using namespace moeq;

MOEQ_API moeq_status moeq_quantize_rtn(const uint16_t *w, int32_t N, int32_t K, int32_t G,
                                       int32_t bits, uint8_t *codes, uint16_t *scales,
                                       uint8_t *zeros, hipStream_t stream) {
  if (!w || !codes || !scales || !zeros) return fail(MOEQ_ERR_INVALID, "quantize_rtn: null pointer");
  if (N <= 0 || K <= 0) return fail(MOEQ_ERR_INVALID, "quantize_rtn: N=%d K=%d must be positive", N, K);
  if (G < 2 || K % G != 0) return fail(MOEQ_ERR_INVALID, "quantize_rtn: G=%d must divide K=%d", G, K);
  if (bits < 2 || bits > 4) return fail(MOEQ_ERR_INVALID, "quantize_rtn: bits=%d not in {2,3,4}", bits);
  const int64_t groups = (int64_t)N * (K / G);
  const int64_t blocks = (groups + 255) / 256;
  if (blocks > 0x7fffffff) return fail(MOEQ_ERR_UNSUPPORTED, "quantize_rtn: too many groups");
  prof_begin("quantize_rtn", stream);
  hipLaunchKernelGGL(quantize_rtn_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, N, K,
                     G, bits, codes, scales, zeros);
  prof_end("quantize_rtn", stream);
  return check_launch("quantize_rtn");
}

MOEQ_API moeq_status moeq_build_lut(const uint16_t *w, const uint8_t *codes4,
                                    const uint16_t *scales, const uint8_t *zeros, int32_t N,
                                    int32_t K, int32_t G, int32_t q, uint16_t *lut,
                                    hipStream_t stream) {
  if (!w || !codes4 || !scales || !zeros || !lut) return fail(MOEQ_ERR_INVALID, "build_lut: null pointer");
  if (N <= 0 || K <= 0) return fail(MOEQ_ERR_INVALID, "build_lut: N=%d K=%d must be positive", N, K);
  if (G < 2 || G > 256 || K % G != 0) return fail(MOEQ_ERR_INVALID, "build_lut: G=%d must divide K=%d and be <= 256", G, K);
  if (q < 2 || q > 4) return fail(MOEQ_ERR_INVALID, "build_lut: q=%d not in {2,3,4}", q);
  const int64_t groups = (int64_t)N * (K / G);
  const int64_t blocks = (groups + 255) / 256;
  if (blocks > 0x7fffffff) return fail(MOEQ_ERR_UNSUPPORTED, "build_lut: too many groups");
  prof_begin("build_lut", stream);
  hipLaunchKernelGGL(build_lut_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, codes4,
                     scales, zeros, N, K, G, q, lut);
  prof_end("build_lut", stream);
  return check_launch("build_lut");
}
