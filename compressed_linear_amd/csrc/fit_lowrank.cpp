// fit_lowrank.cpp -- Naive-LoRA factors on the GPU: the rank-r truncated SVD of
// the residual E = W - W_hat ("SLiM: One-shot Quantization and Sparsity with
// Low-rank Approximation for LLM Weight Compression", review highlights,
// SLiM-LoRA bullet: Naive-LoRA minimises the plain error norm between the
// original and the compressed weight matrix).
//
// Randomized subspace iteration (Halko, Martinsson and Tropp, "Finding
// structure with randomness", 2011): with m = rank + oversample columns and a
// Gaussian start Omega [K, m],
//     Y = E Omega;  repeat q times: Q = orth(Y), Z = orth(E^T Q), Y = E Z;
//     Q = orth(Y);  Z = E^T Q  (so that B = Q^T E = Z^T);
//     B B^T = Z^T Z = W diag(lambda) W^T  (an m x m eigenproblem);
//     U_r = Q W_r, sigma = sqrt(lambda_r), V_r = Z W_r diag(1 / sigma_r).
// The factors take the square root of sigma each (the split the oracle's
// reading fixes): L = V_r diag(sqrt(sigma)) = Z W_r diag(sigma^-1/2),
// R^T = U_r diag(sqrt(sigma)) = Q W_r diag(sigma^1/2).
//
// The products with E (the only large operands) run as rocBLAS sgemm on the
// caller's stream; orth(Y) takes the eigenvectors of the m x m Gram matrix
// Y^T Y (Q = Y V diag(lambda^-1/2), directions below 1e-6 of the largest
// dropped), twice, and every m x m eigenproblem is solved on the host by
// cyclic Jacobi rotations in fp64.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "compressed_linear.h"
#include "internal.h"

namespace cl {
namespace {

constexpr int kMaxCols = 512;  // rank + oversample

// Eigen-decomposition of the symmetric n x n matrix A (row-major, destroyed):
// eigenvalues w descending, eigenvectors the columns of V (row-major n x n).
void jacobi_eigen(std::vector<double>& A, int n, std::vector<double>& w, std::vector<double>& V) {
  V.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) V[(size_t)i * n + i] = 1.0;
  double total = 0.0;
  for (double x : A) total += x * x;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < n; ++p)
      for (int q = p + 1; q < n; ++q) off += A[(size_t)p * n + q] * A[(size_t)p * n + q];
    if (off <= 1e-30 * total || off == 0.0) break;
    for (int p = 0; p < n; ++p) {
      for (int q = p + 1; q < n; ++q) {
        const double apq = A[(size_t)p * n + q];
        if (apq == 0.0) continue;
        const double app = A[(size_t)p * n + p], aqq = A[(size_t)q * n + q];
        const double theta = (aqq - app) / (2.0 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        const double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < n; ++k) {  // columns p, q
          const double akp = A[(size_t)k * n + p], akq = A[(size_t)k * n + q];
          A[(size_t)k * n + p] = c * akp - s * akq;
          A[(size_t)k * n + q] = s * akp + c * akq;
        }
        for (int k = 0; k < n; ++k) {  // rows p, q
          const double apk = A[(size_t)p * n + k], aqk = A[(size_t)q * n + k];
          A[(size_t)p * n + k] = c * apk - s * aqk;
          A[(size_t)q * n + k] = s * apk + c * aqk;
        }
        for (int k = 0; k < n; ++k) {
          const double vkp = V[(size_t)k * n + p], vkq = V[(size_t)k * n + q];
          V[(size_t)k * n + p] = c * vkp - s * vkq;
          V[(size_t)k * n + q] = s * vkp + c * vkq;
        }
      }
    }
  }
  std::vector<int> idx(n);
  for (int i = 0; i < n; ++i) idx[i] = i;
  std::sort(idx.begin(), idx.end(), [&](int a, int b) { return A[(size_t)a * n + a] > A[(size_t)b * n + b]; });
  std::vector<double> V2((size_t)n * n);
  w.resize(n);
  for (int j = 0; j < n; ++j) {
    w[j] = A[(size_t)idx[j] * n + idx[j]];
    for (int i = 0; i < n; ++i) V2[(size_t)i * n + j] = V[(size_t)i * n + idx[j]];
  }
  V.swap(V2);
}

// Gaussian numbers from splitmix64 and the Box-Muller transform.
struct Normal {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  double operator()() {
    const double u1 = ((next() >> 11) + 1.0) * (1.0 / 9007199254740993.0), u2 = (next() >> 11) * (1.0 / 9007199254740992.0);
    return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
  }
};

struct Dev {
  float* p = nullptr;
  ~Dev() {
    if (p) (void)hipFree(p);
  }
};

struct Fit {
  rocblas_handle h = nullptr;
  hipStream_t s = nullptr;
  ~Fit() {
    if (h) rocblas_destroy_handle(h);
  }
  // C (m x n, column-major, ld ldc) = op(A) op(B)
  bool gemm(bool ta, bool tb, int m, int n, int k, const float* A, int lda, const float* B, int ldb, float* C, int ldc) {
    const float one = 1.f, zero = 0.f;
    return rocblas_sgemm(h, ta ? rocblas_operation_transpose : rocblas_operation_none,
                         tb ? rocblas_operation_transpose : rocblas_operation_none, m, n, k, &one, A, lda, B, ldb, &zero, C,
                         ldc) == rocblas_status_success;
  }
  bool to_host(std::vector<float>& h_, const float* d, size_t n) {
    h_.resize(n);
    return hipMemcpyAsync(h_.data(), d, n * 4, hipMemcpyDeviceToHost, s) == hipSuccess && hipStreamSynchronize(s) == hipSuccess;
  }
  bool to_dev(float* d, const std::vector<float>& h_) {
    return hipMemcpyAsync(d, h_.data(), h_.size() * 4, hipMemcpyHostToDevice, s) == hipSuccess &&
           hipStreamSynchronize(s) == hipSuccess;
  }
  // out (n x m, ld n) = an orthonormal basis of the columns of Y (n x m, ld n);
  // T, G: m x m device scratch
  bool orth(const float* Y, float* out, float* tmp, int n, int m, float* G, float* T) {
    const float* in = Y;
    for (int pass = 0; pass < 2; ++pass) {
      float* dst = pass == 0 ? tmp : out;
      std::vector<float> g;
      if (!gemm(true, false, m, m, n, in, n, in, n, G, m) || !to_host(g, G, (size_t)m * m)) return false;
      std::vector<double> A((size_t)m * m), w, V;
      for (int i = 0; i < m; ++i)
        for (int j = 0; j < m; ++j) A[(size_t)i * m + j] = 0.5 * ((double)g[(size_t)j * m + i] + g[(size_t)i * m + j]);
      jacobi_eigen(A, m, w, V);
      std::vector<float> t((size_t)m * m, 0.f);  // column-major T = V diag(lambda^-1/2)
      const double cut = std::max(w[0], 0.0) * 1e-12;
      for (int j = 0; j < m; ++j) {
        const double f = w[j] > cut && w[j] > 0 ? 1.0 / std::sqrt(w[j]) : 0.0;
        for (int i = 0; i < m; ++i) t[(size_t)j * m + i] = (float)(V[(size_t)i * m + j] * f);
      }
      if (!to_dev(T, t) || !gemm(false, false, n, m, m, in, n, T, m, dst, n)) return false;
      in = dst;
    }
    return true;
  }
};

}  // namespace
}  // namespace cl

using namespace cl;

extern "C" cl_status cl_fit_lowrank(const float* E, int32_t N, int32_t K, int32_t rank, int32_t oversample,
                                    int32_t iters, uint64_t seed, float* L, float* R, float* sigma, void* stream) {
  clear_error();
  if (!E || !L || !R) return fail(CL_EINVAL, "E, L and R must not be NULL");
  if (N < 1 || K < 1 || rank < 1 || oversample < 0 || iters < 0 || iters > 100)
    return fail(CL_EINVAL, "N=%d K=%d rank=%d oversample=%d iters=%d out of range", N, K, rank, oversample, iters);
  if (rank > kMaxCols) return fail(CL_EINVAL, "rank %d above %d", rank, kMaxCols);
  const int m = std::min(std::min(rank + oversample, std::min(N, K)), kMaxCols);
  if ((size_t)N * K >= (size_t)1 << 31 || (size_t)N * m * 4 >= (size_t)1 << 31 || (size_t)K * m * 4 >= (size_t)1 << 31)
    return fail(CL_ESIZE, "the residual or a work matrix reaches 2^31 elements or bytes");
  Fit f;
  f.s = static_cast<hipStream_t>(stream);
  if (rocblas_create_handle(&f.h) != rocblas_status_success || rocblas_set_stream(f.h, f.s) != rocblas_status_success)
    return fail(CL_EHIP, "rocBLAS handle");
  Dev Y, Q, Z, Zq, G, T, tmp;
  const size_t nm = (size_t)N * m, km = (size_t)K * m, mm = (size_t)m * m;
  if (hipMalloc(&Y.p, nm * 4) != hipSuccess || hipMalloc(&Q.p, nm * 4) != hipSuccess || hipMalloc(&Z.p, km * 4) != hipSuccess ||
      hipMalloc(&Zq.p, km * 4) != hipSuccess || hipMalloc(&G.p, mm * 4) != hipSuccess || hipMalloc(&T.p, mm * 4) != hipSuccess ||
      hipMalloc(&tmp.p, std::max(nm, km) * 4) != hipSuccess)
    return fail(CL_ENOMEM, "work matrices of the fit");
  // E is row-major [N, K]: the column-major K x N matrix E^T with ld K.
  //   E X   (X: K x m)  = gemm(T, N, N, m, K, E, K, X, K)
  //   E^T X (X: N x m)  = gemm(N, N, K, m, N, E, K, X, N)
  Normal rng{seed};
  std::vector<float> om(km);
  for (auto& v : om) v = (float)rng();
  if (!f.to_dev(Zq.p, om)) return fail(CL_EHIP, "copying the start matrix");
  bool ok = f.gemm(true, false, N, m, K, E, K, Zq.p, K, Y.p, N);
  for (int it = 0; ok && it < iters; ++it) {
    ok = f.orth(Y.p, Q.p, tmp.p, N, m, G.p, T.p) && f.gemm(false, false, K, m, N, E, K, Q.p, N, Z.p, K) &&
         f.orth(Z.p, Zq.p, tmp.p, K, m, G.p, T.p) && f.gemm(true, false, N, m, K, E, K, Zq.p, K, Y.p, N);
  }
  ok = ok && f.orth(Y.p, Q.p, tmp.p, N, m, G.p, T.p) && f.gemm(false, false, K, m, N, E, K, Q.p, N, Z.p, K);
  std::vector<float> g;
  ok = ok && f.gemm(true, false, m, m, K, Z.p, K, Z.p, K, G.p, m) && f.to_host(g, G.p, mm);
  if (!ok) return fail(CL_EHIP, "a product of the subspace iteration failed");
  std::vector<double> A(mm), w, V;
  for (int i = 0; i < m; ++i)
    for (int j = 0; j < m; ++j) A[(size_t)i * m + j] = 0.5 * ((double)g[(size_t)j * m + i] + g[(size_t)i * m + j]);
  jacobi_eigen(A, m, w, V);
  // W_l = W_r diag(sigma^-1/2) and W_r diag(sigma^1/2), m x rank column-major
  // (columns past m, and directions of zero singular value, stay zero)
  std::vector<float> wl((size_t)m * rank, 0.f), wr((size_t)m * rank, 0.f);
  const double smax = std::sqrt(std::max(w[0], 0.0));
  for (int j = 0; j < rank; ++j) {
    const double sj = j < m && w[j] > 0 ? std::sqrt(w[j]) : 0.0;
    if (sigma) sigma[j] = (float)sj;
    if (sj <= smax * 1e-6 || sj == 0.0) continue;
    for (int i = 0; i < m; ++i) {
      wl[(size_t)j * m + i] = (float)(V[(size_t)i * m + j] / std::sqrt(sj));
      wr[(size_t)j * m + i] = (float)(V[(size_t)i * m + j] * std::sqrt(sj));
    }
  }
  // L (row-major K x rank = column-major rank x K) = W_l^T Z^T; R (row-major
  // rank x N = column-major N x rank) = Q W_r
  Dev Wl, Wr;
  if (hipMalloc(&Wl.p, wl.size() * 4) != hipSuccess || hipMalloc(&Wr.p, wr.size() * 4) != hipSuccess)
    return fail(CL_ENOMEM, "work matrices of the fit");
  ok = f.to_dev(Wl.p, wl) && f.to_dev(Wr.p, wr) && f.gemm(true, true, rank, K, m, Wl.p, m, Z.p, K, L, rank) &&
       f.gemm(false, false, N, rank, m, Q.p, N, Wr.p, m, R, N) && hipStreamSynchronize(f.s) == hipSuccess;
  if (!ok) return fail(CL_EHIP, "the factor products failed");
  return CL_OK;
}
