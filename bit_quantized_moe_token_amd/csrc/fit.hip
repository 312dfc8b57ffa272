// Low-rank compensator fitting (data preparation, before the path).
//
// MiLo abstract: a low-rank compensator of each quantized expert block's
// error; TileQ abstract: factors shared by a group of experts.  The factors
// here are the rank-r truncation of the mean quantization residual
//   R = (1/n) sum_m (W_m - s_m (c_m - z_m))
// of n blocks (n = 1: one block's own compensator; n > 1: the factor pair
// shared by a group, which minimizes sum_m ||R_m - U V||_F because
// sum_m ||R_m - X||^2 = sum_m ||R_m - R||^2 + n ||R - X||^2).
//
// The truncation is computed by randomized subspace iteration (the range
// finder of Halko, Martinsson and Tropp, 2011) with a Gaussian test matrix
// the caller draws:
//   Y = R Omega;  q times { Z = orth(R^T orth(Y)); Y = R Z };  Q = orth(Y)
//   B = Q^T R (l x K);  B B^T = E diag(lambda) E^T   (cyclic Jacobi, fp64)
//   U = Q E_r diag(lambda_r^(1/4)),  V = diag(lambda_r^(-1/4)) E_r^T B
// so U V = Q E_r E_r^T B, the rank-r truncation of Q B, with the singular
// values split evenly between U and V (as the oracle splits them).  orth()
// whitens through the eigen-decomposition of the Gram matrix, twice (a
// Cholesky factor breaks down when a planted low-rank residual leaves
// directions of Y at rounding level).  The large products run in one fp32 GEMM
// kernel; the l x l factorizations run on the host in fp64 (the call
// synchronizes its stream for them).
#include <algorithm>
#include <cmath>
#include <vector>

#include "common.hpp"

namespace moeq {

// R[n][k] = (1/n_mat) sum_m (w_m[n][k] - s_m[n][g] * (c_m[n][k] - z_m[n][g])), fp32
__global__ void __launch_bounds__(256)
residual_kernel(const uint16_t *__restrict__ w, const uint8_t *__restrict__ codes,
                const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros, int n_mat, int N, int K,
                int G, float *__restrict__ R) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t NK = (int64_t)N * K;
  if (i >= NK) return;
  const int64_t n = i / K, k = i % K;
  const int64_t gi = n * (K / G) + k / G;
  const int64_t NG = (int64_t)N * (K / G);
  float acc = 0.f;
  for (int m = 0; m < n_mat; ++m) {
    const float wv = (float)__builtin_bit_cast(f16, w[m * NK + i]);
    const float s = (float)__builtin_bit_cast(f16, scales[m * NG + gi]);
    const float cz = (float)((int)codes[m * NK + i] - (int)zeros[m * NG + gi]);
    acc += wv - s * cz;   // s * (c - z) is exact in fp32
  }
  R[i] = acc / (float)n_mat;
}

// C[M][Nc] = sum_k A(m, k) B(k, n), fp32, row-major C; A(m, k) = A[m*lda + k]
// or (TA) A[k*lda + m]; B(k, n) = B[k*ldb + n] or (TB) B[n*ldb + k].
// 64 x 64 tiles, 16-deep K slices staged in LDS, 4 x 4 outputs per thread.
constexpr int kGT = 64, kGK = 16;

template <bool TA, bool TB>
__global__ void __launch_bounds__(256)
gemm_f32_kernel(const float *__restrict__ A, int lda, const float *__restrict__ B, int ldb, float *__restrict__ C,
                int M, int Nc, int Kd) {
  __shared__ float sa[kGK][kGT + 1];
  __shared__ float sb[kGK][kGT + 1];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int m0 = blockIdx.y * kGT, n0 = blockIdx.x * kGT;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < Kd; k0 += kGK) {
    for (int e = tid; e < kGK * kGT; e += 256) {
      const int kk = e / kGT, mm = e % kGT;
      const int m = m0 + mm, k = k0 + kk;
      float va = 0.f;
      if (m < M && k < Kd) va = TA ? A[(int64_t)k * lda + m] : A[(int64_t)m * lda + k];
      sa[kk][mm] = va;
      const int n = n0 + mm;
      float vb = 0.f;
      if (n < Nc && k < Kd) vb = TB ? B[(int64_t)n * ldb + k] : B[(int64_t)k * ldb + n];
      sb[kk][mm] = vb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = sa[kk][ty + 16 * i]; b[i] = sb[kk][tx + 16 * i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty + 16 * i, n = n0 + tx + 16 * j;
      if (m < M && n < Nc) C[(int64_t)m * Nc + n] = acc[i][j];
    }
}

__global__ void __launch_bounds__(256) to_f16_kernel(const float *__restrict__ x, int64_t n, uint16_t *__restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = __builtin_bit_cast(uint16_t, (f16)x[i]);
}

namespace {

// C = op(A) op(B) on the stream (see gemm_f32_kernel).
void gemm(bool ta, bool tb, const float *A, int lda, const float *B, int ldb, float *C, int M, int Nc, int Kd,
          hipStream_t s) {
  const dim3 grid((Nc + kGT - 1) / kGT, (M + kGT - 1) / kGT);
  if (!ta && !tb) hipLaunchKernelGGL((gemm_f32_kernel<false, false>), grid, dim3(256), 0, s, A, lda, B, ldb, C, M, Nc, Kd);
  else if (ta && !tb) hipLaunchKernelGGL((gemm_f32_kernel<true, false>), grid, dim3(256), 0, s, A, lda, B, ldb, C, M, Nc, Kd);
  else if (!ta && tb) hipLaunchKernelGGL((gemm_f32_kernel<false, true>), grid, dim3(256), 0, s, A, lda, B, ldb, C, M, Nc, Kd);
  else hipLaunchKernelGGL((gemm_f32_kernel<true, true>), grid, dim3(256), 0, s, A, lda, B, ldb, C, M, Nc, Kd);
}

// l x l matrix from the device (synchronous on the stream).
bool fetch(const float *d, int l, std::vector<double> &h, hipStream_t s) {
  std::vector<float> f((size_t)l * l);
  if (hipMemcpyAsync(f.data(), d, f.size() * sizeof(float), hipMemcpyDeviceToHost, s) != hipSuccess) return false;
  if (hipStreamSynchronize(s) != hipSuccess) return false;
  h.assign(f.begin(), f.end());
  return true;
}

bool upload(const std::vector<double> &h, float *d, hipStream_t s) {
  std::vector<float> f(h.begin(), h.end());
  if (hipMemcpyAsync(d, f.data(), f.size() * sizeof(float), hipMemcpyHostToDevice, s) != hipSuccess) return false;
  return hipStreamSynchronize(s) == hipSuccess;   // f is freed on return
}

// Eigen-decomposition of a symmetric l x l matrix by cyclic Jacobi
// rotations: on return A's diagonal holds the eigenvalues and E's columns
// the eigenvectors.
void jacobi_eig(std::vector<double> &A, int l, std::vector<double> &E) {
  E.assign((size_t)l * l, 0.0);
  for (int i = 0; i < l; ++i) E[i * l + i] = 1.0;
  for (int sweep = 0; sweep < 60; ++sweep) {
    double off = 0, tot = 0;
    for (int i = 0; i < l; ++i)
      for (int j = 0; j < l; ++j) {
        tot += A[i * l + j] * A[i * l + j];
        if (i != j) off += A[i * l + j] * A[i * l + j];
      }
    if (off <= 1e-26 * tot || off == 0) break;
    for (int p = 0; p < l - 1; ++p)
      for (int q = p + 1; q < l; ++q) {
        const double apq = A[p * l + q];
        if (apq == 0) continue;
        const double theta = (A[q * l + q] - A[p * l + p]) / (2 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1));
        const double c = 1 / std::sqrt(t * t + 1), s = t * c;
        for (int k = 0; k < l; ++k) {   // A <- A J (columns p, q)
          const double akp = A[k * l + p], akq = A[k * l + q];
          A[k * l + p] = c * akp - s * akq;
          A[k * l + q] = s * akp + c * akq;
        }
        for (int k = 0; k < l; ++k) {   // A <- J^T A (rows p, q)
          const double apk = A[p * l + k], aqk = A[q * l + k];
          A[p * l + k] = c * apk - s * aqk;
          A[q * l + k] = s * apk + c * aqk;
        }
        for (int k = 0; k < l; ++k) {   // E <- E J
          const double ekp = E[k * l + p], ekq = E[k * l + q];
          E[k * l + p] = c * ekp - s * ekq;
          E[k * l + q] = s * ekp + c * ekq;
        }
      }
  }
}

// M (l x l, row-major) with X M orthonormal for the Gram matrix G = X^T X:
// M = E diag(lambda^(-1/2)) over the eigenpairs of G above a relative
// threshold (the Gram matrix is accumulated in fp32, so directions below
// ~1e-6 of the largest are noise); the other columns of M are zero, which
// drops those directions from the subspace.
void whiten(std::vector<double> G, int l, std::vector<double> &M) {
  std::vector<double> E;
  jacobi_eig(G, l, E);
  double lmax = 0;
  for (int i = 0; i < l; ++i) lmax = std::max(lmax, G[i * l + i]);
  M.assign((size_t)l * l, 0.0);
  for (int c = 0; c < l; ++c) {
    const double lam = G[c * l + c];
    if (!(lam > 1e-6 * lmax)) continue;
    const double f = 1.0 / std::sqrt(lam);
    for (int i = 0; i < l; ++i) M[i * l + c] = E[i * l + c] * f;
  }
}

struct FitWs {
  size_t R, Y, Y2, Z, Z2, B, S, U32, V32, total;
};

FitWs fit_plan(int N, int K, int r, int l) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  FitWs w;
  size_t off = 0;
  w.R = off; off = al(off + (size_t)N * K * 4);
  w.Y = off; off = al(off + (size_t)N * l * 4);
  w.Y2 = off; off = al(off + (size_t)N * l * 4);
  w.Z = off; off = al(off + (size_t)K * l * 4);
  w.Z2 = off; off = al(off + (size_t)K * l * 4);
  w.B = off; off = al(off + (size_t)l * K * 4);
  w.S = off; off = al(off + (size_t)l * l * 4);
  w.U32 = off; off = al(off + (size_t)N * r * 4);
  w.V32 = off; off = al(off + (size_t)r * K * 4);
  w.total = off;
  return w;
}

constexpr int kFitMaxL = 128;

}  // namespace
}  // namespace moeq

using namespace moeq;

MOEQ_API moeq_status moeq_fit_lowrank_workspace_size(int32_t N, int32_t K, int32_t r, int32_t l, size_t *bytes) {
  if (!bytes) return fail(MOEQ_ERR_INVALID, "fit_lowrank_workspace_size: null output");
  if (N <= 0 || K <= 0 || r < 1 || l < r || l > kFitMaxL || l > N || l > K)
    return fail(MOEQ_ERR_INVALID, "fit_lowrank_workspace_size: N=%d K=%d r=%d l=%d invalid", N, K, r, l);
  *bytes = fit_plan(N, K, r, l).total;
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_fit_lowrank(const uint16_t *w, const uint8_t *codes, const uint16_t *scales,
                                      const uint8_t *zeros, int32_t n_mat, int32_t N, int32_t K, int32_t G,
                                      const float *omega, int32_t l, int32_t r, int32_t power_iters, uint16_t *U,
                                      uint16_t *V, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!w || !codes || !scales || !zeros || !omega || !U || !V)
    return fail(MOEQ_ERR_INVALID, "fit_lowrank: null pointer");
  if (n_mat < 1 || N <= 0 || K <= 0 || G < 2 || K % G != 0)
    return fail(MOEQ_ERR_INVALID, "fit_lowrank: n_mat=%d N=%d K=%d G=%d invalid", n_mat, N, K, G);
  if (r < 1 || l < r || l > kFitMaxL || l > N || l > K)
    return fail(MOEQ_ERR_INVALID, "fit_lowrank: need 1 <= r <= l <= min(N, K, %d) (r=%d l=%d)", kFitMaxL, r, l);
  if (power_iters < 0 || power_iters > 16)
    return fail(MOEQ_ERR_INVALID, "fit_lowrank: power_iters=%d not in 0..16", power_iters);
  if ((int64_t)N * K >= (1ll << 31) / 4)
    return fail(MOEQ_ERR_UNSUPPORTED, "fit_lowrank: N*K=%lld too large", (long long)N * K);
  const FitWs p = fit_plan(N, K, r, l);
  if (!ws || ws_bytes < p.total)
    return fail(MOEQ_ERR_WORKSPACE, "fit_lowrank: workspace has %zu bytes, needs %zu", ws_bytes, p.total);
  uint8_t *wb = static_cast<uint8_t *>(ws);
  float *R = reinterpret_cast<float *>(wb + p.R), *Y = reinterpret_cast<float *>(wb + p.Y);
  float *Y2 = reinterpret_cast<float *>(wb + p.Y2), *Z = reinterpret_cast<float *>(wb + p.Z);
  float *Z2 = reinterpret_cast<float *>(wb + p.Z2), *Bm = reinterpret_cast<float *>(wb + p.B);
  float *S = reinterpret_cast<float *>(wb + p.S), *U32 = reinterpret_cast<float *>(wb + p.U32);
  float *V32 = reinterpret_cast<float *>(wb + p.V32);
  const int64_t NK = (int64_t)N * K;
  hipLaunchKernelGGL(residual_kernel, dim3((unsigned)((NK + 255) / 256)), dim3(256), 0, stream, w, codes, scales,
                     zeros, n_mat, N, K, G, R);
  std::vector<double> Gh, Mh;
  // X (rows x l, in place through tmp) <- X M (whiten), twice
  auto orth = [&](float *X, float *tmp, int rows) -> bool {
    for (int pass = 0; pass < 2; ++pass) {
      gemm(true, false, X, l, X, l, S, l, l, rows, stream);            // X^T X
      if (!fetch(S, l, Gh, stream)) return false;
      whiten(Gh, l, Mh);
      if (!upload(Mh, S, stream)) return false;
      gemm(false, false, X, l, S, l, tmp, rows, l, l, stream);         // X L^-T
      if (hipMemcpyAsync(X, tmp, (size_t)rows * l * 4, hipMemcpyDeviceToDevice, stream) != hipSuccess) return false;
    }
    return true;
  };
  gemm(false, false, R, K, omega, l, Y, N, l, K, stream);              // Y = R Omega
  for (int it = 0; it < power_iters; ++it) {
    if (!orth(Y, Y2, N)) return fail(MOEQ_ERR_HIP, "fit_lowrank: device copy failed");
    gemm(true, false, R, K, Y, l, Z, K, l, N, stream);                 // Z = R^T Y
    if (!orth(Z, Z2, K)) return fail(MOEQ_ERR_HIP, "fit_lowrank: device copy failed");
    gemm(false, false, R, K, Z, l, Y, N, l, K, stream);                // Y = R Z
  }
  if (!orth(Y, Y2, N)) return fail(MOEQ_ERR_HIP, "fit_lowrank: device copy failed");   // Q
  gemm(true, false, Y, l, R, K, Bm, l, K, N, stream);                  // B = Q^T R
  gemm(false, true, Bm, K, Bm, K, S, l, l, K, stream);                 // B B^T
  std::vector<double> A, E;
  if (!fetch(S, l, A, stream)) return fail(MOEQ_ERR_HIP, "fit_lowrank: device copy failed");
  for (int i = 0; i < l; ++i)                                          // symmetrize the fp32 product
    for (int j = i + 1; j < l; ++j) A[i * l + j] = A[j * l + i] = 0.5 * (A[i * l + j] + A[j * l + i]);
  jacobi_eig(A, l, E);
  std::vector<int> order(l);
  for (int i = 0; i < l; ++i) order[i] = i;
  std::sort(order.begin(), order.end(), [&](int a, int b) { return A[a * l + a] > A[b * l + b]; });
  // Pu (l x l, first r columns used) = E_r diag(lambda^(1/4)); Pv (r x l) = diag(lambda^(-1/4)) E_r^T
  std::vector<double> Pu((size_t)l * l, 0.0), Pv((size_t)l * l, 0.0);
  const double lmax = A[order[0] * l + order[0]] > 0 ? A[order[0] * l + order[0]] : 0.0;
  for (int c = 0; c < r; ++c) {
    const int e = order[c];
    const double lam = A[e * l + e];
    const bool ok = lam > 1e-24 * lmax && lam > 0;
    const double up = ok ? std::pow(lam, 0.25) : 0.0, dn = ok ? std::pow(lam, -0.25) : 0.0;
    for (int i = 0; i < l; ++i) {
      Pu[i * l + c] = E[i * l + e] * up;
      Pv[c * l + i] = E[i * l + e] * dn;
    }
  }
  if (!upload(Pu, S, stream)) return fail(MOEQ_ERR_HIP, "fit_lowrank: device copy failed");
  gemm(false, false, Y, l, S, l, U32, N, r, l, stream);                // U = Q Pu[:, :r] (ldb = l)
  if (!upload(Pv, S, stream)) return fail(MOEQ_ERR_HIP, "fit_lowrank: device copy failed");
  gemm(false, false, S, l, Bm, K, V32, r, K, l, stream);               // V = Pv[:r] B
  hipLaunchKernelGGL(to_f16_kernel, dim3((unsigned)(((int64_t)N * r + 255) / 256)), dim3(256), 0, stream, U32,
                     (int64_t)N * r, U);
  hipLaunchKernelGGL(to_f16_kernel, dim3((unsigned)(((int64_t)r * K + 255) / 256)), dim3(256), 0, stream, V32,
                     (int64_t)r * K, V);
  return check_launch("fit_lowrank");
}
