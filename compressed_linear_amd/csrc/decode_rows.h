// decode_rows.h -- batch 1..4 forward: a wavefront per group of rows, lanes along K.
//
// The bandwidth-bound decode path.  A workgroup of four wavefronts owns 4*R
// consecutive rows; wavefront w owns R of them and streams their whole K range:
// in pass p, lane l takes chunk 64p + l of each of its R rows (the row-major
// layout makes that one contiguous 1 KiB load per row), dequantises it through
// the row's LUT table in LDS, and multiplies with the activations of that chunk,
// which it keeps in registers across the R rows.  The 64 lane partials of a
// row are summed with cross-lane shuffles at the end -- no cross-workgroup
// reduction, so no split-K hand-off.
//
// The outliers of a row ("SqueezeLLM: Dense-and-Sparse Quantization",
// Approach: a full-precision CSR matrix) are spread over the 64 lanes, entry
// e going to lane e mod 64 of the row's wavefront: every lane gets the same
// share of a row whatever its length (the page's measured-effects table shows
// a balanced sparse kernel halving generation latency over a standard CSR
// kernel).  The rank-r correction ("SLiM" page, review highlights) is spread
// over the lanes by rank index in the same way.  Both are added to the lane
// partials before the shuffle reduction.
#pragma once
#include <hip/hip_runtime.h>

#include "layer.h"
#include "unpack.h"

namespace cl {

struct RowArgs {
  const uint4* dense;
  const uint8_t* meta;
  const uint16_t* table;
  const int32_t* rowptr;
  const int32_t* col;
  const uint16_t* val;
  const uint8_t* R;
  const uint16_t* Rscale;
  const float* t;
  const void* x;
  float* y;
  int K, N, M, ldx, chunks, rank, group, lr_kind;
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <bool BF16>
__device__ __forceinline__ float x_at(const void* x, int ldx, int m, int k) {
  const uint16_t v = static_cast<const uint16_t*>(x)[(size_t)m * ldx + k];
  if constexpr (BF16) return __uint_as_float((uint32_t)v << 16);
  return (float)__builtin_bit_cast(_Float16, v);
}

template <bool BF16>
__device__ __forceinline__ float mac2r(uint32_t w, uint32_t xv, float acc) {
  if constexpr (!BF16) {
    return __builtin_amdgcn_fdot2(as_h2(w), as_h2(xv), acc, false);
  } else {
    const half2_t h = as_h2(w);
    acc = __builtin_fmaf((float)h.x, __uint_as_float(xv << 16), acc);
    return __builtin_fmaf((float)h.y, __uint_as_float(xv & 0xFFFF0000u), acc);
  }
}

// LDS: the LUT row tables (or the 2:4 selectors) at address 0, then the
// low-rank intermediate t [MB][256] shared by the four wavefronts.
template <int KIND, int MB>
struct RowLds {
  static constexpr int tab = (KIND == K_LUT3 || KIND == K_LUT4) ? 16 * 64 : 32;
  static constexpr int t = tab;
  static constexpr int value = tab + MB * 256;
};

// R = rows per wavefront (the workgroup owns 4*R rows), MB = activation rows (<= 4)
template <int KIND, int MB, bool BF16, int R>
__global__ void __launch_bounds__(256) decode_rows_kernel(RowArgs a) {
  constexpr int SPAN = KindTraits<KIND>::span, P = KindTraits<KIND>::pairs, XD = SPAN / 8;  // uint4 of x per chunk
  static_assert(4 * R <= 16, "row tables hold 16 rows");
  __shared__ uint32_t smem[RowLds<KIND, MB>::value];  // the only LDS object: tables start at address 0
  float* s_t = reinterpret_cast<float*>(smem + RowLds<KIND, MB>::t);
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int row0 = blockIdx.x * 4 * R;
  const int wrow0 = row0 + wave * R;
  build_row_tables<KIND>(smem, a.table, row0, 4 * R, tid, 256);

  float acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[r][m] = 0.f;

  // outliers: the first 64 entries of each row, loaded now, gathered after pass 0
  int e0[R], e1[R], ccol[R];
  float cval[R];
  const bool has_csr = a.rowptr != nullptr;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(wrow0 + r, a.N - 1);
    e0[r] = has_csr ? a.rowptr[row] : 0;
    e1[r] = has_csr && wrow0 + r < a.N ? a.rowptr[row + 1] : e0[r];
    const int e = e0[r] + lane;
    const bool ok = e < e1[r];
    ccol[r] = ok ? a.col[e] : 0;
    cval[r] = ok ? (float)__builtin_bit_cast(_Float16, a.val[e]) : 0.f;
  }
  // low-rank: t [M][rank] into LDS for the four wavefronts (rank <= 256)
  const bool has_lr = a.lr_kind != CL_LR_NONE;
  if (has_lr) {
    for (int i = tid; i < MB * 256; i += 256) {
      const int m = i >> 8, j = i & 255;
      s_t[i] = j < a.rank ? a.t[(m < a.M ? m : a.M - 1) * a.rank + j] : 0.f;
    }
  }
  __syncthreads();

  const int npass = (a.chunks + 63) >> 6;
  const int tail_valid = a.K - (a.chunks - 1) * SPAN;
  const uint4* dbase = a.dense + (size_t)wrow0 * a.chunks + lane;
  const uint2* mbase = reinterpret_cast<const uint2*>(a.meta) + (size_t)wrow0 * a.chunks + lane;
  auto load_codes = [&](uint4 (&w)[R], uint4 (&mw)[R], int p) {
    const bool ok = p * 64 + lane < a.chunks;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      w[r] = ok ? dbase[(size_t)r * a.chunks + p * 64] : make_uint4(0, 0, 0, 0);
      if constexpr (KIND == K_INT4_24) {
        const uint2 v = ok ? mbase[(size_t)r * a.chunks + p * 64] : make_uint2(0, 0);
        mw[r] = make_uint4(v.x, v.y, 0, 0);
      } else {
        mw[r] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  uint4 W[R], MW[R];
  load_codes(W, MW, 0);
  for (int p = 0; p < npass; ++p) {
    const int c = p * 64 + lane;
    // activations of chunk c, all MB rows
    uint32_t xv[MB][P];
    if (c < a.chunks - 1 || (c == a.chunks - 1 && tail_valid == SPAN)) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const uint4* xp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) +
                                                         (size_t)(m < a.M ? m : a.M - 1) * a.ldx + (size_t)c * SPAN);
#pragma unroll
        for (int d = 0; d < XD; ++d) {
          const uint4 v = xp[d];
          xv[m][4 * d] = v.x;
          xv[m][4 * d + 1] = v.y;
          xv[m][4 * d + 2] = v.z;
          xv[m][4 * d + 3] = v.w;
        }
      }
    } else {  // the partial last chunk (pairs past K read as zero) or no chunk
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const uint32_t* xp = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.x) +
                                                               (size_t)(m < a.M ? m : a.M - 1) * a.ldx) +
                             (size_t)c * (SPAN / 2);
#pragma unroll
        for (int j = 0; j < P; ++j) xv[m][j] = (c < a.chunks && 2 * j < tail_valid) ? xp[j] : 0u;
      }
    }
    uint4 Wn[R], MWn[R];
    if (p + 1 < npass) load_codes(Wn, MWn, p + 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t wp[P];
      chunk_pairs<KIND, true>(smem, W[r], MW[r], (uint32_t)((wave * R + r) * 256), 0u, wp);
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < P; ++j) acc[r][m] = mac2r<BF16>(wp[j], xv[m][j], acc[r][m]);
    }
    if (p + 1 < npass) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        W[r] = Wn[r];
        MW[r] = MWn[r];
      }
    }
  }

  // integer formats: the per-row scale multiplies the dense part only
  if constexpr (is_int_kind<KIND>()) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float sc = (float)__builtin_bit_cast(_Float16, a.table[wrow0 + r]);
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[r][m] *= sc;
    }
  }
  // outliers
  if (has_csr) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int m = 0; m < MB; ++m)
        acc[r][m] = __builtin_fmaf(cval[r], x_at<BF16>(a.x, a.ldx, m < a.M ? m : a.M - 1, ccol[r]), acc[r][m]);
      for (int e = e0[r] + 64 + lane; e < e1[r]; e += 64) {
        const float v = (float)__builtin_bit_cast(_Float16, a.val[e]);
        const int cc = a.col[e];
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[r][m] = __builtin_fmaf(v, x_at<BF16>(a.x, a.ldx, m < a.M ? m : a.M - 1, cc), acc[r][m]);
      }
    }
  }
  // low-rank correction: lane j takes rank j, j + 64, ... of each row
  if (has_lr) {
    const int gr = (a.rank + a.group - 1) / a.group;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = wrow0 + r;
      for (int j = lane; j < a.rank; j += 64) {
        float v;
        if (a.lr_kind == CL_LR_INT4) {  // R^T codes [Npad][ceil(r/2)], scales [Npad][ceil(r/g)]
          const uint32_t byte = a.R[(size_t)n * ((a.rank + 1) >> 1) + (j >> 1)];
          const int qv = (int)((byte >> (4 * (j & 1))) & 0xFu) - 8;
          v = (float)qv * (float)__builtin_bit_cast(_Float16, a.Rscale[(size_t)n * gr + j / a.group]);
        } else {  // R^T [Npad][r]
          const uint16_t u = reinterpret_cast<const uint16_t*>(a.R)[(size_t)n * a.rank + j];
          v = a.lr_kind == CL_LR_BF16 ? __uint_as_float((uint32_t)u << 16) : (float)__builtin_bit_cast(_Float16, u);
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[r][m] = __builtin_fmaf(s_t[m * 256 + j], v, acc[r][m]);
      }
    }
  }
  // reduce the 64 lane partials of every (row, activation row)
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const float v = wave_sum(acc[r][m]);
      const int row = wrow0 + r;
      if (lane == 0 && m < a.M && row < a.N) a.y[(size_t)m * a.N + row] = v;
    }
}

template <int KIND, int MB, bool BF16, int R>
static hipError_t launch_rows_t(const RowArgs& a, int Npad, hipStream_t st) {
  hipLaunchKernelGGL((decode_rows_kernel<KIND, MB, BF16, R>), dim3(Npad / (4 * R)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Rows per wavefront: two for one activation row (each activation chunk
// serves two rows; about 120 VGPRs, four waves per SIMD), one for two to four
// activation rows (the activations already fill the registers).
template <int KIND>
hipError_t launch_rows_kind(const RowArgs& a, int Npad, bool bf16, hipStream_t st) {
  if (a.M <= 1)
    return bf16 ? launch_rows_t<KIND, 1, true, 2>(a, Npad, st) : launch_rows_t<KIND, 1, false, 2>(a, Npad, st);
  return bf16 ? launch_rows_t<KIND, 4, true, 1>(a, Npad, st) : launch_rows_t<KIND, 4, false, 1>(a, Npad, st);
}

}  // namespace cl
