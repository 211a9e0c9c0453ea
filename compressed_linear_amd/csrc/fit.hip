// fit.hip -- data-free LUT packing of an fp16 weight matrix on the GPU.
//
// "SqueezeLLM: Dense-and-Sparse Quantization", Approach: each output channel
// (row) gets a non-uniform LUT whose values are k-means centroids of its
// weights, and the outliers leave the dense part for a full-precision CSR
// matrix (0.45 % of the weights in the page's runs).  The sensitivity weighting
// (Fisher information) needs gradients and data; this is the page's
// sensitivity-agnostic variant (its measured-effects table), from weights alone:
//
//   1. outliers: the n_out weights of largest magnitude, ties to the lower
//      row-major index -- a two-pass radix select over the 15-bit magnitude
//      (high 8 bits, then low 7), per-row counts of the threshold value and a
//      scan that hands each row its share of the ties;
//   2. per row (one workgroup): Lloyd's iterations in one dimension over the
//      row's dense weights from 2^b evenly spaced starting points; a weight
//      joins the nearest centroid (the lower one on a tie), a centroid becomes
//      the mean of its weights (kept when it has none), until no centroid moves
//      or max_iter rounds;
//   3. LUT = centroids rounded to fp16; every dense weight takes its nearest LUT
//      value's code (lower on a tie); an outlier's position takes the code
//      nearest to 0 and its CSR value is fp16(w - lut[code]).
//
// All arithmetic that decides a result is exact or rounded once in a fixed
// order: fp16 weights are integer multiples of 2^-24, so the cluster sums are
// kept as 64-bit integers (exact in any order for |w| < 8192, K <= 28672), a
// centroid is sum / count in fp64, boundaries are (c_j + c_j+1) / 2 in fp64.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"
#include "layout.h"

namespace cl {

namespace {

constexpr int kFitThreads = 256;
constexpr int kFitMaxK = 28672;  // the row and its mask bits, with the static LDS, fit 64 KiB

// Work buffer layout (bytes), for N rows.
struct FitWork {
  static constexpr size_t hist1 = 0;          // u32 [256]: magnitude >> 7
  static constexpr size_t hist2 = 1024;       // u32 [128]: magnitude & 127 within the selected bucket
  static constexpr size_t scal = 1536;        // i64 [8]: bucket, need, T, r, bad flag
  static constexpr size_t rows = 1600;        // per row: gt u32 [N], eq u32 [N], eqbase i64 [N]
  __host__ __device__ static size_t gt(int) { return rows; }
  __host__ __device__ static size_t eq(int N) { return rows + (size_t)N * 4; }
  __host__ __device__ static size_t eqbase(int N) { return (rows + (size_t)N * 8 + 7) & ~(size_t)7; }
  __host__ __device__ static size_t bytes(int N) { return eqbase(N) + (size_t)N * 8; }
};
enum { S_BUCKET = 0, S_NEED, S_T, S_R, S_BAD, S_ITERS };

__device__ __forceinline__ uint32_t mag(uint16_t h) { return h & 0x7FFFu; }

// fp16 bits -> the weight as an integer multiple of 2^-24 (exact).
__device__ __forceinline__ long long f16_fixed(uint16_t h) {
  const uint32_t e = (h >> 10) & 31u, m = h & 0x3FFu;
  const long long q = e ? (long long)(m | 0x400u) << (e - 1) : (long long)m;
  return (h & 0x8000u) ? -q : q;
}

// fp64 -> fp16 bits, nearest with ties to even, for values inside the fp16
// range (the centroids and outlier residuals of weights below 8192).
__device__ __forceinline__ uint16_t f64_to_f16_rne(double d) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(d);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const unsigned long long a = u & 0x7FFFFFFFFFFFFFFFull;
  if (a == 0) return (uint16_t)sign;
  const int e = (int)(a >> 52) - 1023;
  const unsigned long long m = (a & 0xFFFFFFFFFFFFFull) | 0x10000000000000ull;  // 53-bit significand
  if (e >= 16) return (uint16_t)(sign | 0x7C00u);
  // keep the bits of weight >= 2^-24 (subnormal) or the top 11 (normal)
  const int shift = e >= -14 ? 42 : 28 - e;
  if (shift > 63) return (uint16_t)sign;
  unsigned long long q = m >> shift;
  const unsigned long long rem = m & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (e >= -14) {
    int ee = e;
    if (q == 2048) { q = 1024; ++ee; }
    if (ee >= 16) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | ((uint32_t)(ee + 15) << 10) | ((uint32_t)q & 0x3FFu));
  }
  return (uint16_t)(sign | (uint32_t)q);  // q == 1024 is the smallest normal
}

__device__ __forceinline__ double f16_to_f64(uint16_t h) { return (double)(float)__builtin_bit_cast(_Float16, h); }

// ---- 1. radix select of the outlier threshold ----
__global__ void __launch_bounds__(256) fit_hist_kernel(const uint16_t* __restrict__ W, long long total, int pass,
                                                      uint8_t* __restrict__ work) {
  __shared__ uint32_t h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  long long* sc = reinterpret_cast<long long*>(work + FitWork::scal);
  const uint32_t bucket = pass ? (uint32_t)sc[S_BUCKET] : 0u;
  uint32_t bad = 0;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const uint32_t u = mag(W[i]);
    if (pass == 0) {
      bad |= u >= 0x7000u;  // |w| >= 8192, inf or NaN
      atomicAdd(&h[u >> 7], 1u);
    } else if ((u >> 7) == bucket) {
      atomicAdd(&h[u & 127u], 1u);
    }
  }
  if (bad) atomicOr(reinterpret_cast<unsigned long long*>(&sc[S_BAD]), 1ull);
  __syncthreads();
  uint32_t* g = reinterpret_cast<uint32_t*>(work + (pass ? FitWork::hist2 : FitWork::hist1));
  if ((int)threadIdx.x < (pass ? 128 : 256) && h[threadIdx.x]) atomicAdd(&g[threadIdx.x], h[threadIdx.x]);
}

// One thread: walk the histogram from the largest magnitude down until n_out is reached.
__global__ void fit_select_kernel(long long n_out, int pass, uint8_t* __restrict__ work) {
  long long* sc = reinterpret_cast<long long*>(work + FitWork::scal);
  const uint32_t* g = reinterpret_cast<const uint32_t*>(work + (pass ? FitWork::hist2 : FitWork::hist1));
  const int nb = pass ? 128 : 256;
  long long need = pass ? sc[S_NEED] : n_out;
  if (need <= 0) {  // no outliers: a threshold above every magnitude
    sc[S_BUCKET] = 256;
    sc[S_NEED] = 0;
    sc[S_T] = 0x8000;
    sc[S_R] = 0;
    return;
  }
  int b = nb - 1;
  for (; b > 0; --b) {
    if ((long long)g[b] >= need) break;
    need -= g[b];
  }
  if (pass == 0) {
    sc[S_BUCKET] = b;
    sc[S_NEED] = need;
  } else {
    sc[S_T] = (sc[S_BUCKET] << 7) | b;
    sc[S_R] = need;  // weights of magnitude T that become outliers, lowest indices first
  }
}

// ---- per-row counts above / at the threshold ----
__global__ void __launch_bounds__(256) fit_rowstat_kernel(const uint16_t* __restrict__ W, int K, uint8_t* __restrict__ work,
                                                          int N) {
  const long long* sc = reinterpret_cast<const long long*>(work + FitWork::scal);
  const uint32_t T = (uint32_t)sc[S_T];
  const uint16_t* row = W + (size_t)blockIdx.x * K;
  uint32_t gt = 0, eq = 0;
  for (int k = threadIdx.x; k < K; k += 256) {
    const uint32_t u = mag(row[k]);
    gt += u > T;
    eq += u == T;
  }
  __shared__ uint32_t sg[256], se[256];
  sg[threadIdx.x] = gt;
  se[threadIdx.x] = eq;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      sg[threadIdx.x] += sg[threadIdx.x + s];
      se[threadIdx.x] += se[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    reinterpret_cast<uint32_t*>(work + FitWork::gt(N))[blockIdx.x] = sg[0];
    reinterpret_cast<uint32_t*>(work + FitWork::eq(N))[blockIdx.x] = se[0];
  }
}

// One workgroup: eqbase = exclusive scan of the rows' threshold counts, each
// row's outlier count, row_ptr = exclusive scan of those (row_ptr[N] = n_out).
__global__ void __launch_bounds__(1024) fit_scan_kernel(int N, uint8_t* __restrict__ work, int32_t* __restrict__ row_ptr) {
  const long long* sc = reinterpret_cast<const long long*>(work + FitWork::scal);
  const long long r = sc[S_R];
  const uint32_t* gt = reinterpret_cast<const uint32_t*>(work + FitWork::gt(N));
  const uint32_t* eq = reinterpret_cast<const uint32_t*>(work + FitWork::eq(N));
  long long* eqbase = reinterpret_cast<long long*>(work + FitWork::eqbase(N));
  __shared__ long long se[1024], so[1024];
  long long carry_e = 0, carry_o = 0;
  for (int base = 0; base < N; base += 1024) {
    const int n = base + (int)threadIdx.x;
    const long long e = n < N ? (long long)eq[n] : 0;
    se[threadIdx.x] = e;
    __syncthreads();
    for (int s = 1; s < 1024; s <<= 1) {  // inclusive scan
      const long long v = (int)threadIdx.x >= s ? se[threadIdx.x - s] : 0;
      __syncthreads();
      se[threadIdx.x] += v;
      __syncthreads();
    }
    const long long ebase = carry_e + se[threadIdx.x] - e;
    long long take = r - ebase;
    take = take < 0 ? 0 : (take > e ? e : take);
    const long long o = n < N ? (long long)gt[n] + take : 0;
    if (n < N) eqbase[n] = ebase;
    so[threadIdx.x] = o;
    __syncthreads();
    for (int s = 1; s < 1024; s <<= 1) {
      const long long v = (int)threadIdx.x >= s ? so[threadIdx.x - s] : 0;
      __syncthreads();
      so[threadIdx.x] += v;
      __syncthreads();
    }
    if (n < N) row_ptr[n] = (int32_t)(carry_o + so[threadIdx.x] - o);
    const long long te = se[1023], to = so[1023];
    __syncthreads();
    carry_e += te;
    carry_o += to;
  }
  if (threadIdx.x == 0) row_ptr[N] = (int32_t)carry_o;
}

// Exclusive prefix of a per-thread flag over the workgroup in thread order,
// plus the workgroup's total.  `tmp`: 4 ints of LDS.
__device__ __forceinline__ int wg_prefix(bool f, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(f);
  const int below = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) tmp[wave] = __popcll(bal);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? tmp[w] : 0;
    tot += tmp[w];
  }
  __syncthreads();
  *total = tot;
  return before + below;
}

// ---- 2 and 3: one workgroup per row ----
template <int NC>
__global__ void __launch_bounds__(kFitThreads) fit_rows_kernel(const uint16_t* __restrict__ W, int N, int K, int max_iter,
                                                               int n_out,
                                                               const uint8_t* __restrict__ work,
                                                               const int32_t* __restrict__ row_ptr,
                                                               uint8_t* __restrict__ codes, uint16_t* __restrict__ lut,
                                                               int32_t* __restrict__ col, uint16_t* __restrict__ val) {
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  uint16_t* v16 = reinterpret_cast<uint16_t*>(dyn);                       // the row, [K]
  uint32_t* outb = reinterpret_cast<uint32_t*>(dyn + ((size_t)K * 2 + 15) / 16 * 16);  // outlier bits, [K/32]
  __shared__ double cen[NC];
  __shared__ float bnd32[NC];
  __shared__ unsigned long long wsum[4][NC];
  __shared__ uint32_t wcnt[4][NC];
  __shared__ int tmp[4];
  __shared__ int s_changed;
  __shared__ uint32_t s_mn, s_mx;
  __shared__ int s_any;

  const int n = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long* sc = reinterpret_cast<const long long*>(work + FitWork::scal);
  const uint32_t T = (uint32_t)sc[S_T];
  const long long r = sc[S_R];
  const long long eqbase = reinterpret_cast<const long long*>(work + FitWork::eqbase(N))[n];
  const uint16_t* row = W + (size_t)n * K;
  for (int k = tid; k < K; k += kFitThreads) v16[k] = row[k];
  for (int i = tid; i < (K + 31) / 32; i += kFitThreads) outb[i] = 0;
  if (tid == 0) {
    s_mn = 0xFFFFFFFFu;
    s_mx = 0;
    s_any = 0;
  }
  __syncthreads();

  // outliers in index order: tiles of 256 consecutive weights, thread t on weight 256 i + t
  const int base_out = row_ptr[n];
  int eq_run = 0, out_run = 0;
  for (int k0 = 0; k0 < K; k0 += kFitThreads) {
    const int k = k0 + tid;
    const uint32_t u = k < K ? mag(v16[k]) : 0u;
    const bool eq = k < K && u == T;
    int eq_tot;
    const int eq_rank = eq_run + wg_prefix(eq, tmp, &eq_tot);
    const bool out = k < K && (u > T || (eq && eqbase + eq_rank < r));
    int out_tot;
    const int out_rank = out_run + wg_prefix(out, tmp, &out_tot);
    if (out) {
      atomicOr(&outb[k >> 5], 1u << (k & 31));
      if (base_out + out_rank < n_out) col[base_out + out_rank] = k;  // always, by the counts; bounds kept anyway
    }
    eq_run += eq_tot;
    out_run += out_tot;
  }
  __syncthreads();

  // range of the dense weights: order-preserving keys of fp16 values (-0 taken as +0)
  auto key = [](uint16_t h) -> uint32_t {
    h = h == 0x8000u ? (uint16_t)0 : h;
    return (h & 0x8000u) ? (uint32_t)(~h & 0xFFFFu) : (uint32_t)(h | 0x8000u);
  };
  auto unkey = [](uint32_t kk) -> uint16_t { return (kk & 0x8000u) ? (uint16_t)(kk & 0x7FFFu) : (uint16_t)(~kk & 0xFFFFu); };
  uint32_t mn = 0xFFFFFFFFu, mx = 0;
  bool any = false;
  for (int k = tid; k < K; k += kFitThreads) {
    if ((outb[k >> 5] >> (k & 31)) & 1u) continue;
    const uint32_t kk = key(v16[k]);
    mn = kk < mn ? kk : mn;
    mx = kk > mx ? kk : mx;
    any = true;
  }
  if (any) {
    atomicMin(&s_mn, mn);
    atomicMax(&s_mx, mx);
    atomicOr(&s_any, 1);
  }
  __syncthreads();

  if (tid < NC) {
    if (s_any) {
      const double dmn = f16_to_f64(unkey(s_mn)), dmx = f16_to_f64(unkey(s_mx));
      cen[tid] = dmn + ((dmx - dmn) * (double)(2 * tid + 1)) / (double)(2 * NC);
    } else {
      cen[tid] = 0.0;
    }
  }
  __syncthreads();

  int done = 0;
  for (int it = 0; it < max_iter && s_any; ++it) {
    ++done;
    // v > b holds exactly when v > RD32(b) for an fp32 v (no fp32 lies strictly
    // between RD32(b) and b), so the assignment compares in fp32
    if (tid < NC - 1) bnd32[tid] = __double2float_rd((cen[tid] + cen[tid + 1]) * 0.5);
    if (tid < 4 * NC) {
      (&wsum[0][0])[tid] = 0;
      (&wcnt[0][0])[tid] = 0;
    }
    if (tid == 0) s_changed = 0;
    __syncthreads();
    float b[NC - 1];
#pragma unroll
    for (int j = 0; j < NC - 1; ++j) b[j] = bnd32[j];
    for (int k = tid; k < K; k += kFitThreads) {
      if ((outb[k >> 5] >> (k & 31)) & 1u) continue;
      const uint16_t h = v16[k];
      const float v = (float)__builtin_bit_cast(_Float16, h);
      int idx = 0;
#pragma unroll
      for (int j = 0; j < NC - 1; ++j) idx += v > b[j];
      // per-wavefront cluster sums: exact integers, so their order is free
      atomicAdd(&wsum[wave][idx], (unsigned long long)f16_fixed(h));
      atomicAdd(&wcnt[wave][idx], 1u);
    }
    __syncthreads();
    if (tid < NC) {
      const long long s = (long long)(wsum[0][tid] + wsum[1][tid] + wsum[2][tid] + wsum[3][tid]);
      const int c = (int)(wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid]);
      if (c > 0) {
        const double nc = ((double)s / (double)c) * (1.0 / 16777216.0);
        if (nc != cen[tid]) {
          cen[tid] = nc;
          s_changed = 1;
        }
      }
    }
    __syncthreads();
    if (!s_changed) break;
  }

  if (tid == 0 && done)
    atomicAdd(reinterpret_cast<unsigned long long*>(const_cast<uint8_t*>(work) + FitWork::scal + S_ITERS * 8),
              (unsigned long long)done);
  // LUT and codes
  __shared__ uint16_t l16[NC];
  __shared__ double lb[NC];
  if (tid < NC) {
    l16[tid] = f64_to_f16_rne(cen[tid]);
    lut[(size_t)n * NC + tid] = l16[tid];
  }
  __syncthreads();
  if (tid < NC - 1) lb[tid] = (f16_to_f64(l16[tid]) + f16_to_f64(l16[tid + 1])) * 0.5;
  __syncthreads();
  double b[NC - 1];
#pragma unroll
  for (int j = 0; j < NC - 1; ++j) b[j] = lb[j];
  uint8_t* crow = codes + (size_t)n * K;
  for (int k = tid; k < K; k += kFitThreads) {
    const bool out = (outb[k >> 5] >> (k & 31)) & 1u;
    const double v = out ? 0.0 : f16_to_f64(v16[k]);
    int idx = 0;
#pragma unroll
    for (int j = 0; j < NC - 1; ++j) idx += b[j] < v;
    crow[k] = (uint8_t)idx;
  }
  // outlier values, in the same index order as their columns
  int idx0 = 0;
  {
    double t = 0.0;
#pragma unroll
    for (int j = 0; j < NC - 1; ++j) idx0 += b[j] < t;
  }
  out_run = 0;
  for (int k0 = 0; k0 < K; k0 += kFitThreads) {
    const int k = k0 + tid;
    const bool out = k < K && ((outb[k >> 5] >> (k & 31)) & 1u);
    int out_tot;
    const int out_rank = out_run + wg_prefix(out, tmp, &out_tot);
    if (out && base_out + out_rank < n_out)
      val[base_out + out_rank] = f64_to_f16_rne(f16_to_f64(v16[k]) - f16_to_f64(l16[idx0]));
    out_run += out_tot;
  }
}

// ---- integer formats: data-free mask and SLiM-Quant clip search, one workgroup per row ----
//
// "SLiM" page, review highlights: symmetric quantization that clips the weights
// before rounding to nearest, the clipping threshold found by a grid search (the
// page's probabilistic formulation has lost its equations; read here as the
// plain squared error of the row's kept weights).  Rebuttal "Unstructured vs.
// 2:4 Sparsity" and "Compressing Large Language Models by Joint Sparsification
// and Quantization", Approach: 2:4 and unstructured masks; without activations
// the mask keeps the largest magnitudes (ties to the lower index).
//   scale candidates s_i = fp16((i * max|w|) / (qmax * G)), i = 1..G (fp64 division,
//   then nearest-even fp16); codes q = clamp(rint(w / s_i), -qmax, qmax); the
//   error sum of (w - s_i q)^2 over the kept weights is an exact 128-bit integer
//   in units of 2^-48; the smallest wins, the lower i on a tie.
typedef unsigned __int128 u128;

template <int QMAX>
__global__ void __launch_bounds__(kFitThreads) fit_int_kernel(const uint16_t* __restrict__ W, int K, int mask, int grid,
                                                              int8_t* __restrict__ qvals, uint16_t* __restrict__ row_scale,
                                                              uint8_t* __restrict__ keep_out, unsigned long long* __restrict__ bad) {
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  uint16_t* v16 = reinterpret_cast<uint16_t*>(dyn);
  uint32_t* keepb = reinterpret_cast<uint32_t*>(dyn + ((size_t)K * 2 + 15) / 16 * 16);
  __shared__ uint32_t hist[256];
  __shared__ u128 red[4];
  __shared__ int tmp[4];
  __shared__ uint32_t s_T, s_mag;
  __shared__ int s_r, s_bucket;
  const int n = blockIdx.x, tid = threadIdx.x;
  const uint16_t* row = W + (size_t)n * K;
  uint32_t nonfinite = 0;
  for (int k = tid; k < K; k += kFitThreads) {
    v16[k] = row[k];
    nonfinite |= (row[k] & 0x7C00u) == 0x7C00u;
  }
  for (int i = tid; i < (K + 31) / 32; i += kFitThreads) keepb[i] = 0;
  if (nonfinite) atomicOr(bad, 1ull);
  if (tid == 0) s_mag = 0;
  __syncthreads();

  // ---- mask ----
  if (mask == CL_MASK_2_4) {
    for (int g = tid; g < K / 4; g += kFitThreads) {
      uint32_t a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = mag(v16[4 * g + t]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        int beaten = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) beaten += (a[u] > a[t]) || (a[u] == a[t] && u < t);
        if (beaten < 2) atomicOr(&keepb[(4 * g + t) >> 5], 1u << ((4 * g + t) & 31));
      }
    }
  } else if (mask == CL_MASK_BITMAP) {
    // the floor(K/2) largest magnitudes: radix select (high 8 bits, low 7), ties by index
    const int want = K / 2;
    for (int pass = 0; pass < 2; ++pass) {
      hist[tid] = 0;
      __syncthreads();
      for (int k = tid; k < K; k += kFitThreads) {
        const uint32_t u = mag(v16[k]);
        if (pass == 0) atomicAdd(&hist[u >> 7], 1u);
        else if ((int)(u >> 7) == s_bucket) atomicAdd(&hist[u & 127u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int need = pass == 0 ? want : s_r, b = pass == 0 ? 255 : 127;
        if (need <= 0) {
          s_bucket = 256;
          s_T = 0x8000u;
          s_r = 0;
        } else {
          for (; b > 0; --b) {
            if ((int)hist[b] >= need) break;
            need -= (int)hist[b];
          }
          if (pass == 0) {
            s_bucket = b;
            s_r = need;
          } else {
            s_T = ((uint32_t)s_bucket << 7) | (uint32_t)b;
            s_r = need;
          }
        }
      }
      __syncthreads();
      if (s_bucket == 256) break;
    }
    const uint32_t T = s_T;
    const int r = s_r;
    int eq_run = 0;
    for (int k0 = 0; k0 < K; k0 += kFitThreads) {
      const int k = k0 + tid;
      const uint32_t u = k < K ? mag(v16[k]) : 0u;
      const bool eq = k < K && u == T;
      int tot;
      const int rank = eq_run + wg_prefix(eq, tmp, &tot);
      if (k < K && (u > T || (eq && rank < r))) atomicOr(&keepb[k >> 5], 1u << (k & 31));
      eq_run += tot;
    }
  } else {
    for (int i = tid; i < K / 32; i += kFitThreads) keepb[i] = 0xFFFFFFFFu;
    if (tid == 0 && (K & 31)) keepb[K / 32] = (1u << (K & 31)) - 1u;
  }
  __syncthreads();
  auto kept = [&](int k) -> bool { return (keepb[k >> 5] >> (k & 31)) & 1u; };
  uint32_t mx = 0;
  for (int k = tid; k < K; k += kFitThreads)
    if (kept(k)) mx = max(mx, mag(v16[k]));
  if (mx) atomicMax(&s_mag, mx);
  __syncthreads();
  const double m = f16_to_f64((uint16_t)s_mag);

  // ---- clip search ----
  u128 best = ~(u128)0;
  int best_i = 0;
  uint16_t best_s = 0;
  for (int i = 1; i <= grid; ++i) {
    const uint16_t s16 = f64_to_f16_rne(((double)i * m) / (double)(QMAX * grid));
    if ((s16 & 0x7FFFu) == 0) continue;  // uniform: every thread skips
    const double sd = f16_to_f64(s16);
    const long long S = f16_fixed(s16);
    u128 acc = 0;
    for (int k = tid; k < K; k += kFitThreads) {
      if (!kept(k)) continue;
      const uint16_t h = v16[k];
      double qd = rint(f16_to_f64(h) / sd);
      qd = qd > QMAX ? QMAX : (qd < -QMAX ? -QMAX : qd);
      const long long d = f16_fixed(h) - S * (long long)qd;
      const unsigned long long ad = (unsigned long long)(d < 0 ? -d : d);
      acc += (u128)ad * ad;
    }
    // 128-bit sum over the wavefront (two 64-bit halves and the carry), then the four wavefronts
    unsigned long long lo = (unsigned long long)acc, hi = (unsigned long long)(acc >> 64);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long lo2 = __shfl_xor(lo, o, 64), hi2 = __shfl_xor(hi, o, 64);
      const unsigned long long sl = lo + lo2;
      hi = hi + hi2 + (sl < lo ? 1ull : 0ull);
      lo = sl;
    }
    if ((tid & 63) == 0) red[tid >> 6] = ((u128)hi << 64) | lo;
    __syncthreads();
    if (tid == 0) {
      const u128 tot = red[0] + red[1] + red[2] + red[3];
      if (tot < best) {
        best = tot;
        best_i = i;
        best_s = s16;
      }
    }
    __syncthreads();
  }
  __shared__ uint16_t s_best;
  if (tid == 0) {
    s_best = best_i ? best_s : (uint16_t)0;
    row_scale[n] = s_best;
  }
  __syncthreads();
  const uint16_t s16 = s_best;
  const double sd = f16_to_f64(s16);
  int8_t* qrow = qvals + (size_t)n * K;
  uint8_t* krow = keep_out ? keep_out + (size_t)n * K : nullptr;
  for (int k = tid; k < K; k += kFitThreads) {
    int q = 0;
    if (kept(k) && (s16 & 0x7FFFu)) {
      double qd = rint(f16_to_f64(v16[k]) / sd);
      q = (int)(qd > QMAX ? QMAX : (qd < -QMAX ? -QMAX : qd));
    }
    qrow[k] = (int8_t)q;
    if (krow) krow[k] = kept(k) ? 1 : 0;
  }
}

// ---- AbsMax int4 groups of a low-rank factor, one thread per (group, column) ----
// "SLiM" page, review highlights: the adapters are quantized with an AbsMax group
// scheme, group size 128.  F is [R, C] (L [K, r]: groups along K; R [r, N]:
// groups along r); scale = fp16(max|v| / 7) (fp64 division, nearest-even fp16),
// q = clamp(rint(v / scale), -8, 7) in fp64; an all-zero group: scale 0, q 0.
template <bool BF16>
__global__ void __launch_bounds__(256) fit_absmax_kernel(const uint16_t* __restrict__ F, int R, int C, int group,
                                                         int8_t* __restrict__ q, uint16_t* __restrict__ scale) {
  const int cb = (C + 255) / 256, g = (int)(blockIdx.x / cb), c = (int)(blockIdx.x % cb) * 256 + (int)threadIdx.x;
  if (c >= C) return;
  const int r0 = g * group, r1 = min(R, r0 + group);
  auto val = [&](int r) -> double {
    const uint16_t h = F[(size_t)r * C + c];
    return BF16 ? (double)__uint_as_float((uint32_t)h << 16) : f16_to_f64(h);
  };
  double m = 0.0;
  for (int r = r0; r < r1; ++r) m = fmax(m, fabs(val(r)));
  const uint16_t s16 = f64_to_f16_rne(m / 7.0);
  scale[(size_t)g * C + c] = s16;
  const double sd = f16_to_f64(s16);
  for (int r = r0; r < r1; ++r) {
    double qd = 0.0;
    if (sd > 0.0) {
      qd = rint(val(r) / sd);
      qd = qd > 7.0 ? 7.0 : (qd < -8.0 ? -8.0 : qd);
    }
    q[(size_t)r * C + c] = (int8_t)qd;
  }
}

}  // namespace

}  // namespace cl

using namespace cl;

namespace cl {
namespace {

__global__ void fit_zero_kernel(unsigned long long* __restrict__ p, int n8) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n8) p[i] = 0ull;
}

cl_status fit_lut_check(const uint16_t* W, int32_t N, int32_t K, int32_t bits, int64_t n_out, int32_t max_iter,
                        uint8_t* codes, uint16_t* lut, int32_t* row_ptr, int32_t* col, uint16_t* val) {
  if (N < 1 || K < 1) return fail(CL_EINVAL, "N and K must be >= 1");
  if (K > kFitMaxK || N > (1 << 24)) return fail(CL_ESIZE, "the fitter takes K <= %d and N <= 2^24", kFitMaxK);
  if (bits != 3 && bits != 4) return fail(CL_EINVAL, "bits must be 3 or 4");
  if (max_iter < 1) return fail(CL_EINVAL, "max_iter must be >= 1");
  const long long total = (long long)N * K;
  if (n_out < 0 || n_out > total || n_out > 0x7FFFFFFFLL) return fail(CL_EINVAL, "n_out out of range");
  if (!W || !codes || !lut || !row_ptr || (n_out > 0 && (!col || !val))) return fail(CL_EINVAL, "a required pointer is NULL");
  return CL_OK;
}

// The fit of a checked call, with its scratch at `wk` (FitWork::bytes(N) bytes,
// 8-byte aligned): histograms and scalars are cleared by a kernel (no memset
// node), the kernels run, and the call waits for the scalars it reports.
cl_status fit_lut_run(const uint16_t* W, int32_t N, int32_t K, int32_t bits, int64_t n_out, int32_t max_iter,
                      uint8_t* codes, uint16_t* lut, int32_t* row_ptr, int32_t* col, uint16_t* val, uint8_t* wk,
                      hipStream_t s, int64_t* total_iters) {
  const long long total = (long long)N * K;
  const int hb = (int)(total / 256 / 8 + 1 > 2048 ? 2048 : total / 256 / 8 + 1);
  static_assert(FitWork::rows % 8 == 0, "the cleared head is whole words");
  hipLaunchKernelGGL(fit_zero_kernel, dim3((unsigned)ceil_div(FitWork::rows / 8, 256)), dim3(256), 0, s,
                     reinterpret_cast<unsigned long long*>(wk), (int)(FitWork::rows / 8));  // histograms and scalars
  hipLaunchKernelGGL(fit_hist_kernel, dim3(hb), dim3(256), 0, s, W, total, 0, wk);
  hipLaunchKernelGGL(fit_select_kernel, dim3(1), dim3(1), 0, s, (long long)n_out, 0, wk);
  hipLaunchKernelGGL(fit_hist_kernel, dim3(hb), dim3(256), 0, s, W, total, 1, wk);
  hipLaunchKernelGGL(fit_select_kernel, dim3(1), dim3(1), 0, s, (long long)n_out, 1, wk);
  hipLaunchKernelGGL(fit_rowstat_kernel, dim3(N), dim3(256), 0, s, W, K, wk, N);
  hipLaunchKernelGGL(fit_scan_kernel, dim3(1), dim3(1024), 0, s, N, wk, row_ptr);
  const size_t lds = ((size_t)K * 2 + 15) / 16 * 16 + ((size_t)K + 31) / 32 * 4;
  if (bits == 3)
    hipLaunchKernelGGL(fit_rows_kernel<8>, dim3(N), dim3(kFitThreads), lds, s, W, N, K, max_iter, (int)n_out, wk, row_ptr,
                       codes, lut, col, val);
  else
    hipLaunchKernelGGL(fit_rows_kernel<16>, dim3(N), dim3(kFitThreads), lds, s, W, N, K, max_iter, (int)n_out, wk, row_ptr,
                       codes, lut, col, val);
  hipError_t e = hipGetLastError();
  long long sc[8] = {};
  if (e == hipSuccess) e = hipMemcpyAsync(sc, wk + FitWork::scal, sizeof(sc), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(CL_EHIP, "fit failed: %s", hipGetErrorString(e));
  if (sc[S_BAD]) return fail(CL_EINVAL, "a weight is not finite or its magnitude is 8192 or more (outputs are not valid)");
  if (total_iters) *total_iters = sc[S_ITERS];
  return CL_OK;
}

// Scratch of the fitter variant that allocates nothing: one array per device,
// held until the process ends; its device address is looked up once per
// device (the name is only a host-side stand-in) and kept.  Calls on one
// device share it.
constexpr size_t kFitScratchBytes = (size_t)2 << 20;
// rows it serves: FitWork::bytes(N) = 1600 + 16 N <= 2 MiB
constexpr int kFitNoallocMaxRows = (int)((kFitScratchBytes - FitWork::rows) / 16);
static_assert(FitWork::rows % 8 == 0 && FitWork::rows + 16 * (size_t)kFitNoallocMaxRows <= kFitScratchBytes,
              "the scratch holds the work of kFitNoallocMaxRows rows");
__device__ __align__(256) uint8_t scratch[kFitScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

cl_status scratch_of_current_device(uint8_t** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CL_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(CL_EUNSUPPORTED, "device %d beyond the %d this library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (es != hipSuccess || !p) return fail(CL_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(es));
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return CL_OK;
}

}  // namespace
}  // namespace cl

extern "C" size_t cl_fit_lut_work_bytes(int32_t N, int32_t K) {
  if (N < 1 || K < 1) return 0;
  return FitWork::bytes(N);
}

extern "C" cl_status cl_fit_lut(const uint16_t* W, int32_t N, int32_t K, int32_t bits, int64_t n_out, int32_t max_iter,
                                uint8_t* codes, uint16_t* lut, int32_t* row_ptr, int32_t* col, uint16_t* val,
                                void* work, void* stream, int64_t* total_iters) {
  clear_error();
  cl_status st = fit_lut_check(W, N, K, bits, n_out, max_iter, codes, lut, row_ptr, col, val);
  if (st != CL_OK) return st;
  if (!work) return fail(CL_EINVAL, "a required pointer is NULL");
  if (reinterpret_cast<uintptr_t>(work) % 8) return fail(CL_EINVAL, "work must be 8-byte aligned");
  return fit_lut_run(W, N, K, bits, n_out, max_iter, codes, lut, row_ptr, col, val, static_cast<uint8_t*>(work),
                     static_cast<hipStream_t>(stream), total_iters);
}

extern "C" cl_status cl_fit_lut_noalloc(const uint16_t* W, int32_t N, int32_t K, int32_t bits, int64_t n_out,
                                        int32_t max_iter, uint8_t* codes, uint16_t* lut, int32_t* row_ptr, int32_t* col,
                                        uint16_t* val, void* stream, int64_t* total_iters) {
  clear_error();
  cl_status st = fit_lut_check(W, N, K, bits, n_out, max_iter, codes, lut, row_ptr, col, val);
  if (st != CL_OK) return st;
  if (N > kFitNoallocMaxRows || FitWork::bytes(N) > kFitScratchBytes)
    return fail(CL_ESIZE, "the fitter without a work buffer takes N <= %d rows (its scratch is %zu bytes)",
                kFitNoallocMaxRows, kFitScratchBytes);
  uint8_t* wk = nullptr;
  st = scratch_of_current_device(&wk);
  if (st != CL_OK) return st;
  return fit_lut_run(W, N, K, bits, n_out, max_iter, codes, lut, row_ptr, col, val, wk, static_cast<hipStream_t>(stream),
                     total_iters);
}

extern "C" cl_status cl_fit_int(const uint16_t* W, int32_t N, int32_t K, int32_t bits, int32_t mask, int32_t grid,
                                int8_t* qvals, uint16_t* row_scale, uint8_t* keep, void* work, void* stream) {
  clear_error();
  if (N < 1 || K < 1) return fail(CL_EINVAL, "N and K must be >= 1");
  if (K > kFitMaxK || N > (1 << 24)) return fail(CL_ESIZE, "the fitter takes K <= %d and N <= 2^24", kFitMaxK);
  if (bits != 4 && bits != 8) return fail(CL_EINVAL, "bits must be 4 or 8");
  if (mask != CL_MASK_NONE && mask != CL_MASK_2_4 && mask != CL_MASK_BITMAP) return fail(CL_EINVAL, "unknown mask %d", mask);
  if (mask == CL_MASK_2_4 && (bits != 4 || K % 4)) return fail(CL_EUNSUPPORTED, "2:4 needs bits = 4 and K % 4 == 0");
  if (mask == CL_MASK_BITMAP && bits != 8) return fail(CL_EUNSUPPORTED, "the unstructured mask needs bits = 8");
  if (grid < 1 || grid > 4096) return fail(CL_EINVAL, "grid must be in [1, 4096]");
  if (!W || !qvals || !row_scale || !work || (mask != CL_MASK_NONE && !keep))
    return fail(CL_EINVAL, "a required pointer is NULL");
  if (reinterpret_cast<uintptr_t>(work) % 8) return fail(CL_EINVAL, "work must be 8-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned long long* bad = static_cast<unsigned long long*>(work);
  hipError_t e = hipMemsetAsync(bad, 0, 8, s);
  const size_t lds = ((size_t)K * 2 + 15) / 16 * 16 + ((size_t)K + 31) / 32 * 4;
  if (e == hipSuccess) {
    if (bits == 4)
      hipLaunchKernelGGL(fit_int_kernel<7>, dim3(N), dim3(kFitThreads), lds, s, W, K, mask, grid, qvals, row_scale, keep, bad);
    else
      hipLaunchKernelGGL(fit_int_kernel<127>, dim3(N), dim3(kFitThreads), lds, s, W, K, mask, grid, qvals, row_scale, keep,
                         bad);
    e = hipGetLastError();
  }
  unsigned long long flag = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&flag, bad, 8, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(CL_EHIP, "fit failed: %s", hipGetErrorString(e));
  if (flag) return fail(CL_EINVAL, "a weight is not finite (outputs are not valid)");
  return CL_OK;
}

extern "C" cl_status cl_quant_absmax(const uint16_t* F, int32_t R, int32_t C, int32_t group, int32_t bf16, int8_t* q,
                                     uint16_t* scale, void* stream) {
  clear_error();
  if (R < 1 || C < 1 || group < 1) return fail(CL_EINVAL, "R, C and group must be >= 1");
  if ((long long)R * C > (1ll << 40)) return fail(CL_ESIZE, "the factor is too large");
  if (!F || !q || !scale) return fail(CL_EINVAL, "a required pointer is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const long long blocks = ceil_div(C, 256) * ceil_div(R, group);
  if (blocks > 0x7FFFFFFFLL) return fail(CL_ESIZE, "the factor is too large");
  const dim3 grid((unsigned)blocks);
  if (bf16)
    hipLaunchKernelGGL(fit_absmax_kernel<true>, grid, dim3(256), 0, s, F, R, C, group, q, scale);
  else
    hipLaunchKernelGGL(fit_absmax_kernel<false>, grid, dim3(256), 0, s, F, R, C, group, q, scale);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CL_EHIP, "launch failed: %s", hipGetErrorString(e));
  return CL_OK;
}
