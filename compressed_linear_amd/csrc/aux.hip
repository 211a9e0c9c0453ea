// aux.hip -- activation preparation, the low-rank prologue and the debug dequantiser.
#include <hip/hip_runtime.h>

#include "layer.h"
#include "lowrank.h"
#include "unpack.h"

namespace cl {

// ---------------------------------------------------------------------------
// x' = clamp(x, -c, c), then x'[k] * f[k] on the scaled channels, copied to a
// row stride Kx (a multiple of 8) with a zero tail.
// Clamp: activation editor of "Compressing Large Language Models by Joint
// Sparsification and Quantization", Approach (one clamp value per layer).
// Scaling: "SLiM" page, rebuttal section "Output Error Minimization in
// SLiM-Quant" (the activations of the salient channels divided by alpha; the
// layer stores f = 1/alpha per channel, 1 elsewhere).  x * f is exact in fp32
// (at most 11 + 11 significant bits, f a normal fp16 <= 1) and is rounded once,
// to nearest-even, to the activation type.
// ---------------------------------------------------------------------------
// One thread per eight consecutive channels of one row (grid: K groups x M rows);
// rows of 16-byte loads when K is a multiple of 8, element loads otherwise.
template <bool BF16>
__global__ void __launch_bounds__(256) prep_x_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ xp, int K,
                                                     int Kx, int has_clamp, float c, const uint16_t* __restrict__ xs) {
  const int m = blockIdx.y, k = ((int)blockIdx.x * 256 + (int)threadIdx.x) * 8;
  if (k >= Kx) return;
  const uint16_t* xr = x + (size_t)m * K;
  uint4 v, f = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
  if ((K & 7) == 0) {  // Kx == K: k + 8 <= K, 16-byte aligned rows
    v = *reinterpret_cast<const uint4*>(xr + k);
    if (xs) f = *reinterpret_cast<const uint4*>(xs + k);
  } else {
    uint32_t e[4], g[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k0 = k + 2 * j, k1 = k0 + 1;
      e[j] = (k0 < K ? (uint32_t)xr[k0] : 0u) | ((k1 < K ? (uint32_t)xr[k1] : 0u) << 16);
      g[j] = (xs && k0 < K ? (uint32_t)xs[k0] : 0x3C00u) | ((xs && k1 < K ? (uint32_t)xs[k1] : 0x3C00u) << 16);
    }
    v = make_uint4(e[0], e[1], e[2], e[3]);
    f = make_uint4(g[0], g[1], g[2], g[3]);
  }
  if (has_clamp) v = clamp_act8<BF16>(v, c);  // +-c is exact in the activation type (checked by the packer)
  if (xs) v = scale_act8<BF16>(v, f);
  *reinterpret_cast<uint4*>(xp + (size_t)m * Kx + k) = v;
}

hipError_t launch_prep_x(const Layer& L, int M, const void* x, hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(L.Kx / 8, 256), (unsigned)M);
  const float c = (float)__builtin_bit_cast(_Float16, L.h.act_clamp);
  if (L.h.x_dtype == CL_ACT_BF16)
    hipLaunchKernelGGL(prep_x_kernel<true>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), L.xprep, L.h.K, L.Kx, L.h.has_clamp, c, L.xscale);
  else
    hipLaunchKernelGGL(prep_x_kernel<false>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), L.xprep, L.h.K, L.Kx, L.h.has_clamp, c, L.xscale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Low-rank prologue t = x' L_hat (fp32 [M, rank]), "SLiM" page, review
// highlights (SLiM-LoRA; AbsMax int4 groups of 128 along K for L).
// L is stored transposed ([rank][K]), so workgroup j reads rank column j as one
// contiguous stream: thread i takes 8 consecutive k at a time, every 2048-th
// k, and the 256 partial dot products are summed in a fixed order (shuffles
// within a wavefront, then the four wavefronts in order).  No workgroup
// depends on another: t[m][j] is written by workgroup j alone.
// ---------------------------------------------------------------------------
struct LrArgs {
  const uint16_t* x;
  int ldx, M, K, rank, group, lr_kind;
  const uint8_t* L;    // L^T
  const uint16_t* Ls;  // L^T scales [rank][ceil(K/group)]
  float* t;            // [M][rank]
};

template <int MB, bool BF16>
__global__ void __launch_bounds__(256) lr_prologue_kernel(LrArgs a) {
  __shared__ float red[4][MB];
  const int j = blockIdx.x, m0 = blockIdx.y * MB, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, gk = (K + a.group - 1) / a.group;
  float acc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = 0.f;
  for (int k0 = tid * 8; k0 < K; k0 += 256 * 8) {
    float l[8];
    if (a.lr_kind == CL_LR_INT4) {
      const uint8_t* lp = a.L + (size_t)j * ((K + 1) >> 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = k0 + i;
        float v = 0.f;
        if (k < K) {
          const int qv = (int)((lp[k >> 1] >> (4 * (k & 1))) & 0xF) - 8;
          v = (float)qv * (float)__builtin_bit_cast(_Float16, a.Ls[(size_t)j * gk + k / a.group]);
        }
        l[i] = v;
      }
    } else {
      const uint16_t* lp = reinterpret_cast<const uint16_t*>(a.L) + (size_t)j * K;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = k0 + i;
        const uint16_t u = k < K ? lp[k] : (uint16_t)0;
        l[i] = a.lr_kind == CL_LR_BF16 ? __uint_as_float((uint32_t)u << 16) : (float)__builtin_bit_cast(_Float16, u);
      }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const uint16_t* xr = a.x + (size_t)min(m0 + m, a.M - 1) * a.ldx;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = k0 + i;
        const uint16_t u = k < K ? xr[k] : (uint16_t)0;
        const float xf = BF16 ? __uint_as_float((uint32_t)u << 16) : (float)__builtin_bit_cast(_Float16, u);
        acc[m] = __builtin_fmaf(xf, l[i], acc[m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    float v = acc[m];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) red[wave][m] = v;
  }
  __syncthreads();
  if (tid < MB && m0 + tid < a.M) {
    const float v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    a.t[(size_t)(m0 + tid) * a.rank + j] = v;
  }
}

template <int MODE, int MT, bool BF16>
__global__ void __launch_bounds__(256) lr_split_kernel(LrSplitArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LrScratch<MODE, MT>::bytes];
  lr_split_block<MODE, MT, BF16, false>(a, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.y, smem);
}

template <int MODE, int MT>
static void launch_lr_split(const LrSplitArgs& a, bool bf, dim3 grid, hipStream_t st) {
  if (bf) hipLaunchKernelGGL((lr_split_kernel<MODE, MT, true>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((lr_split_kernel<MODE, MT, false>), grid, dim3(256), 0, st, a);
}

LrSplitArgs lowrank_split_args(const Layer& L, int M, const void* x) {
  LrSplitArgs s = {};  // flag = NULL: a kernel of its own
  s.x = static_cast<const uint16_t*>(x);
  s.ldx = (x == L.xprep) ? L.Kx : L.h.K;
  s.M = M;
  s.rank = L.h.rank;
  s.rpad = L.lr_rpad;
  s.S = L.lr_S;
  s.group = L.h.group > 0 ? L.h.group : 1;
  s.Kl = L.lr_S * kLrSlice;
  s.lk = L.lr_lk;
  s.ls = L.lr_ls;
  s.part = L.lr_part;
  s.cnt = L.lr_cnt;
  s.t = L.t;
  s.done = L.lr_cnt + 64;
  s.ntiles = (L.lr_rpad / 64) * (int)ceil_div(M, lowrank_tile_m(M));
  return s;
}

hipError_t launch_lowrank_prologue(const Layer& L, int M, const void* x, hipStream_t stream) {
  if (L.lr_mode >= 0 && M <= kMaxDecodeM) {
    const LrSplitArgs s = lowrank_split_args(L, M, x);
    const int MT = lowrank_tile_m(M);
    const dim3 grid((unsigned)L.lr_S, (unsigned)(L.lr_rpad / 64), (unsigned)ceil_div(M, MT));
    const bool bf = L.h.x_dtype == CL_ACT_BF16;
#define LRS(mode, mt) \
  if (L.lr_mode == mode && MT == mt) launch_lr_split<mode, mt>(s, bf, grid, stream);
    LRS(0, 1) LRS(0, 2) LRS(0, 4) LRS(1, 1) LRS(1, 2) LRS(1, 4)
#undef LRS
    return hipGetLastError();
  }
  LrArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.ldx = (x == L.xprep) ? L.Kx : L.h.K;
  a.M = M;
  a.K = L.h.K;
  a.rank = L.h.rank;
  a.group = L.h.group > 0 ? L.h.group : 1;
  a.lr_kind = L.h.lr;
  a.L = L.L;
  a.Ls = L.Lscale;
  a.t = L.t;
  const bool bf = L.h.x_dtype == CL_ACT_BF16;
  const int MB = M <= 1 ? 1 : M <= 4 ? 4 : M <= 16 ? 16 : 32;
  dim3 grid(a.rank, (unsigned)ceil_div(M, MB));
#define LRL(mb)                                                                                \
  if (MB == mb) {                                                                              \
    if (bf) hipLaunchKernelGGL((lr_prologue_kernel<mb, true>), grid, dim3(256), 0, stream, a); \
    else hipLaunchKernelGGL((lr_prologue_kernel<mb, false>), grid, dim3(256), 0, stream, a);   \
  }
  LRL(1) LRL(4) LRL(16) LRL(32)
#undef LRL
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Debug dequantisation: the same chunk_pairs() and tables as the forward,
// stored to fp16.  Non-bitmap formats go through the row tables of the
// batch-1..4 kernel (a wavefront per row, lanes along K); the bitmap format
// through the tile kernel's per-lane staging (a lane per row).
// ---------------------------------------------------------------------------
template <int KIND>
__global__ void __launch_bounds__(256) debug_rows_kernel(const Layer L, uint16_t* __restrict__ D16) {
  constexpr int SPAN = KindTraits<KIND>::span, P = KindTraits<KIND>::pairs;
  __shared__ uint32_t smem[(KIND == K_LUT3 || KIND == K_LUT4) ? 4 * row_table_bytes<KIND>() / 4 : 32];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = blockIdx.x * 4, n = row0 + wave;
  const int K = L.h.K, C = L.h.chunks;
  build_row_tables<KIND>(smem, reinterpret_cast<const uint16_t*>(L.table), row0, 4, tid, 256);
  __syncthreads();
  if (n >= L.h.N) return;
  const float scale =
      is_int_kind<KIND>() ? (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(L.table)[n]) : 1.f;
  for (int c = lane; c < C; c += 64) {
    const uint4 w = reinterpret_cast<const uint4*>(L.dense)[(size_t)n * C + c];
    uint4 mw = make_uint4(0, 0, 0, 0);
    if constexpr (KIND == K_INT4_24) {
      const uint2 mv = reinterpret_cast<const uint2*>(L.meta)[(size_t)n * C + c];
      mw = make_uint4(mv.x, mv.y, 0, 0);
    }
    uint32_t wp[P];
    chunk_pairs<KIND, true>(smem, w, mw, (uint32_t)(wave * row_table_bytes<KIND>()), 0u, wp);
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int k = c * SPAN + 2 * j;
      const half2_t h = as_h2(wp[j]);
      _Float16 v0 = h.x, v1 = h.y;
      if (is_int_kind<KIND>()) {
        v0 = (_Float16)((float)h.x * scale);
        v1 = (_Float16)((float)h.y * scale);
      }
      if (k < K) D16[(size_t)n * K + k] = __builtin_bit_cast(uint16_t, v0);
      if (k + 1 < K) D16[(size_t)n * K + k + 1] = __builtin_bit_cast(uint16_t, v1);
    }
  }
}

__global__ void __launch_bounds__(64) debug_bitmap_kernel(const Layer L, uint16_t* __restrict__ D16) {
  constexpr int SPAN = KindTraits<K_INT8_BM>::span, P = KindTraits<K_INT8_BM>::pairs;
  __shared__ uint32_t smem[kBmSelDwords + 64 * kBmSlot];
  const int tile = blockIdx.x, lane = threadIdx.x, n = tile * 64 + lane;
  const int K = L.h.K, N = L.h.N, C = L.h.chunks;
  build_tables<K_INT8_BM>(smem, reinterpret_cast<const uint16_t*>(L.table), tile, lane, 64);
  __syncthreads();
  const float scale = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(L.table)[n]);
  const uint32_t slot_base = (uint32_t)(kBmSelDwords + lane * kBmSlot) * 4u;
  long long nz_cur = n < N ? L.nzoff[n] : 0;
  for (int c = 0; c < C; ++c) {
    const uint4 w = reinterpret_cast<const uint4*>(L.meta)[(size_t)n * C + c];
    const int cnt = __builtin_popcount(w.x) + __builtin_popcount(w.y) + __builtin_popcount(w.z) + __builtin_popcount(w.w);
    const uint32_t mis = (uint32_t)(nz_cur & 3);
    const uint32_t* s4 = reinterpret_cast<const uint32_t*>(L.dense + nz_cur - mis);
    const int nd = (cnt + (int)mis + 3) >> 2;
    for (int d = 0; d < nd; ++d) smem[slot_base / 4 + d] = s4[d];
    nz_cur += cnt;
    uint32_t wp[P];
    chunk_pairs<K_INT8_BM>(smem, w, make_uint4(0, 0, 0, 0), 0u, slot_base + mis, wp);
    if (n < N) {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int k = c * SPAN + 2 * j;
        const half2_t h = as_h2(wp[j]);
        const _Float16 v0 = (_Float16)((float)h.x * scale), v1 = (_Float16)((float)h.y * scale);
        if (k < K) D16[(size_t)n * K + k] = __builtin_bit_cast(uint16_t, v0);
        if (k + 1 < K) D16[(size_t)n * K + k + 1] = __builtin_bit_cast(uint16_t, v1);
      }
    }
  }
}

__global__ void fill_u16_kernel(uint16_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

__global__ void debug_sparse_kernel(const int32_t* rp, const int32_t* col, const uint16_t* val, uint16_t* S16, int N, int K) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  for (int p = rp[n]; p < rp[n + 1]; ++p) S16[(size_t)n * K + col[p]] = val[p];
}

// L_hat [K][r] and R_hat [r][N] in fp32 from the transposed device factors.
__global__ void debug_lowrank_kernel(const Layer L, float* L32, float* R32) {
  const int K = L.h.K, N = L.h.N, r = L.h.rank, g = L.h.group > 0 ? L.h.group : 1;
  const int hr = (r + 1) / 2, hk = (K + 1) / 2, gk = (K + g - 1) / g, gr = (r + g - 1) / g;
  const size_t nl = (size_t)K * r, nr = (size_t)r * N;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nl + nr; i += (size_t)gridDim.x * blockDim.x) {
    if (i < nl) {
      if (!L32) continue;
      const int k = (int)(i / r), j = (int)(i % r);
      float v;
      if (L.h.lr == CL_LR_INT4) {
        const int qv = (int)((L.L[(size_t)j * hk + (k >> 1)] >> (4 * (k & 1))) & 0xF) - 8;
        v = (float)qv * (float)__builtin_bit_cast(_Float16, L.Lscale[(size_t)j * gk + k / g]);
      } else {
        const uint16_t u = reinterpret_cast<const uint16_t*>(L.L)[(size_t)j * K + k];
        v = L.h.lr == CL_LR_BF16 ? __uint_as_float((uint32_t)u << 16) : (float)__builtin_bit_cast(_Float16, u);
      }
      L32[i] = v;
    } else {
      if (!R32) continue;
      const size_t ii = i - nl;
      const int j = (int)(ii / N), n = (int)(ii % N);
      float v;
      if (L.h.lr == CL_LR_INT4) {
        const int qv = (int)((L.R[(size_t)n * hr + (j >> 1)] >> (4 * (j & 1))) & 0xF) - 8;
        v = (float)qv * (float)__builtin_bit_cast(_Float16, L.Rscale[(size_t)n * gr + j / g]);
      } else {
        const uint16_t u = reinterpret_cast<const uint16_t*>(L.R)[(size_t)n * r + j];
        v = L.h.lr == CL_LR_BF16 ? __uint_as_float((uint32_t)u << 16) : (float)__builtin_bit_cast(_Float16, u);
      }
      R32[ii] = v;
    }
  }
}

hipError_t launch_debug(const Layer& L, uint16_t* D16, uint16_t* S16, float* L32, float* R32, hipStream_t stream) {
  const cl_blob_header& h = L.h;
  dim3 grid_rows(L.Npad / 4);
  switch (h.dense) {
    case CL_DENSE_LUT3: hipLaunchKernelGGL(debug_rows_kernel<K_LUT3>, grid_rows, dim3(256), 0, stream, L, D16); break;
    case CL_DENSE_LUT4: hipLaunchKernelGGL(debug_rows_kernel<K_LUT4>, grid_rows, dim3(256), 0, stream, L, D16); break;
    case CL_DENSE_INT4:
      if (h.mask == CL_MASK_2_4)
        hipLaunchKernelGGL(debug_rows_kernel<K_INT4_24>, grid_rows, dim3(256), 0, stream, L, D16);
      else
        hipLaunchKernelGGL(debug_rows_kernel<K_INT4>, grid_rows, dim3(256), 0, stream, L, D16);
      break;
    default:
      if (h.mask == CL_MASK_BITMAP)
        hipLaunchKernelGGL(debug_bitmap_kernel, dim3(h.n_tiles), dim3(64), 0, stream, L, D16);
      else
        hipLaunchKernelGGL(debug_rows_kernel<K_INT8>, grid_rows, dim3(256), 0, stream, L, D16);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t plane = (size_t)h.N * h.K;
  hipLaunchKernelGGL(fill_u16_kernel, dim3(1024), dim3(256), 0, stream, S16, plane);
  if (h.nnz > 0)
    hipLaunchKernelGGL(debug_sparse_kernel, dim3((unsigned)ceil_div(h.N, 256)), dim3(256), 0, stream, L.rowptr, L.col,
                       L.val, S16, h.N, h.K);
  if (h.lr != CL_LR_NONE && h.rank > 0 && (L32 || R32))
    hipLaunchKernelGGL(debug_lowrank_kernel, dim3(1024), dim3(256), 0, stream, L, L32, R32);
  return hipGetLastError();
}

}  // namespace cl
