// aux.hip -- activation preparation, the low-rank prologue and the debug dequantiser.
#include <hip/hip_runtime.h>

#include "layer.h"
#include "unpack.h"

namespace cl {

// ---------------------------------------------------------------------------
// x' = clamp(x, -c, c), copied to a row stride Kx (even) with a zero tail.
// Activation editor of "Compressing Large Language Models by Joint
// Sparsification and Quantization", Approach: one clamp value per layer.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ void prep_x_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ xp, int M, int K, int Kx,
                              int has_clamp, float c) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)M * Kx;
  if (i >= total) return;
  const int m = (int)(i / Kx), k = (int)(i % Kx);
  uint16_t v = 0;
  if (k < K) {
    v = x[(size_t)m * K + k];
    if (has_clamp) {
      float f = BF16 ? __uint_as_float((uint32_t)v << 16) : (float)__builtin_bit_cast(_Float16, v);
      f = fminf(fmaxf(f, -c), c);  // +-c is exact in the activation type (checked by the packer)
      v = BF16 ? (uint16_t)(__float_as_uint(f) >> 16) : __builtin_bit_cast(uint16_t, (_Float16)f);
    }
  }
  xp[i] = v;
}

hipError_t launch_prep_x(const Layer& L, int M, const void* x, hipStream_t stream) {
  const size_t total = (size_t)M * L.Kx;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  const float c = (float)__builtin_bit_cast(_Float16, L.h.act_clamp);
  if (L.h.x_dtype == CL_ACT_BF16)
    hipLaunchKernelGGL(prep_x_kernel<true>, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), L.xprep, M, L.h.K, L.Kx, L.h.has_clamp, c);
  else
    hipLaunchKernelGGL(prep_x_kernel<false>, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), L.xprep, M, L.h.K, L.Kx, L.h.has_clamp, c);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Low-rank prologue t = x' L_hat (fp32 [M, rank]), "SLiM" page, review
// highlights (SLiM-LoRA; AbsMax int4 groups of 128 along K for L).
// Workgroup (b, mb) sums k in [b*KS, (b+1)*KS) for rows mb*MB.. of x'; thread
// (j, q) takes rank column j and every nq-th k.  Partial sums are reduced in
// a fixed order; the last workgroup of an m-block adds the K blocks in order.
// ---------------------------------------------------------------------------
struct LrArgs {
  const uint16_t* x;
  int ldx, M, K, rank, group, lr_kind, KS, nblocks, half_r;
  const uint8_t* L;
  const uint16_t* Ls;
  float* tpart;   // [nblocks][M][rank]
  float* t;       // [M][rank]
  uint32_t* counters;  // one per m-block
};

template <int MB, bool BF16>
__global__ void __launch_bounds__(256) lr_prologue_kernel(LrArgs a) {
  __shared__ float red[256 * MB];
  __shared__ int s_last;
  const int b = blockIdx.x, mb = blockIdx.y, tid = threadIdx.x;
  const int m0 = mb * MB;
  const int r = a.rank, nq = 256 / r;
  const int j = tid % r, q = tid / r;
  const int k0 = b * a.KS, k1 = min(a.K, k0 + a.KS);
  float acc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = 0.f;
  if (q < nq) {
    for (int k = k0 + q; k < k1; k += nq) {
      float l;
      if (a.lr_kind == CL_LR_INT4) {
        const uint32_t byte = a.L[(size_t)k * a.half_r + (j >> 1)];
        const int qv = (int)((byte >> (4 * (j & 1))) & 0xFu) - 8;
        l = (float)qv * (float)__builtin_bit_cast(_Float16, a.Ls[(size_t)(k / a.group) * r + j]);
      } else {
        const uint16_t v = reinterpret_cast<const uint16_t*>(a.L)[(size_t)k * r + j];
        l = a.lr_kind == CL_LR_BF16 ? __uint_as_float((uint32_t)v << 16) : (float)__builtin_bit_cast(_Float16, v);
      }
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const int mm = min(m0 + m, a.M - 1);
        const uint16_t xv = a.x[(size_t)mm * a.ldx + k];
        const float xf = BF16 ? __uint_as_float((uint32_t)xv << 16) : (float)__builtin_bit_cast(_Float16, xv);
        acc[m] = __builtin_fmaf(xf, l, acc[m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MB; ++m) red[m * 256 + tid] = acc[m];
  __syncthreads();
  for (int i = tid; i < MB * r; i += 256) {
    const int m = i / r, jj = i % r;
    float v = 0.f;
    for (int qq = 0; qq < nq; ++qq) v += red[m * 256 + qq * r + jj];
    if (m0 + m < a.M) a.tpart[((size_t)b * a.M + m0 + m) * r + jj] = v;
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&a.counters[mb], 1u) == (uint32_t)(a.nblocks - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int i = tid; i < MB * r; i += 256) {
    const int m = i / r, jj = i % r;
    if (m0 + m >= a.M) continue;
    float v = 0.f;
    for (int bb = 0; bb < a.nblocks; ++bb)
      v += __builtin_nontemporal_load(a.tpart + ((size_t)bb * a.M + m0 + m) * r + jj);
    a.t[(size_t)(m0 + m) * r + jj] = v;
  }
  if (tid == 0) a.counters[mb] = 0u;
}

hipError_t launch_lowrank_prologue(const Layer& L, int M, const void* x, hipStream_t stream) {
  LrArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.ldx = (x == L.xprep) ? L.Kx : L.h.K;
  a.M = M;
  a.K = L.h.K;
  a.rank = L.h.rank;
  a.group = L.h.group > 0 ? L.h.group : 1;
  a.lr_kind = L.h.lr;
  a.nblocks = L.lr_blocks;
  a.KS = (int)ceil_div(L.h.K, L.lr_blocks);
  a.half_r = (int)ceil_div(L.h.rank, 2);
  a.L = L.L;
  a.Ls = L.Lscale;
  a.tpart = L.tpart;
  a.t = L.t;
  a.counters = L.counters + L.h.n_tiles;
  const bool bf = L.h.x_dtype == CL_ACT_BF16;
  const int MB = M <= 1 ? 1 : M <= 4 ? 4 : M <= 16 ? 16 : 32;
  dim3 grid(a.nblocks, (unsigned)ceil_div(M, MB));
#define LRL(mb)                                                                          \
  if (MB == mb) {                                                                        \
    if (bf) hipLaunchKernelGGL((lr_prologue_kernel<mb, true>), grid, dim3(256), 0, stream, a); \
    else hipLaunchKernelGGL((lr_prologue_kernel<mb, false>), grid, dim3(256), 0, stream, a);   \
  }
  LRL(1) LRL(4) LRL(16) LRL(32)
#undef LRL
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Debug dequantisation: the same chunk_pairs() as the forward, stored to fp16.
// One wavefront per (tile, chunk block); the bitmap format walks whole rows.
// ---------------------------------------------------------------------------
template <int KIND>
__global__ void __launch_bounds__(64) debug_dense_kernel(const Layer L, uint16_t* __restrict__ D16, int cblk) {
  constexpr int SPAN = KindTraits<KIND>::span, P = KindTraits<KIND>::pairs;
  constexpr int TAB = KIND == K_INT8_BM ? (kBmSelDwords + 64 * kBmSlot)
                                        : (KindTraits<KIND>::tab_dwords > 0 ? KindTraits<KIND>::tab_dwords : 1);
  __shared__ uint32_t smem[TAB];
  const int tile = blockIdx.x, lane = threadIdx.x, n = tile * 64 + lane;
  const int K = L.h.K, N = L.h.N, C = L.h.chunks;
  build_tables<KIND>(smem, reinterpret_cast<const uint16_t*>(L.table), tile, lane, 64);
  __syncthreads();
  const int cb = KIND == K_INT8_BM ? 0 : blockIdx.y * cblk;
  const int ce = KIND == K_INT8_BM ? C : min(C, cb + cblk);
  const uint32_t lanebase = (uint32_t)lane * 4u;
  const bool int_kind = KIND >= K_INT4;
  const float scale = int_kind ? (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(L.table)[n]) : 1.f;
  const uint32_t slot_base = (uint32_t)(kBmSelDwords + lane * kBmSlot) * 4u;
  long long nz_cur = (KIND == K_INT8_BM && n < N) ? L.nzoff[n] : 0;
  for (int c = cb; c < ce; ++c) {
    uint4 w, mw = make_uint4(0, 0, 0, 0);
    uint32_t sb = 0;
    if constexpr (KIND == K_INT8_BM) {
      w = reinterpret_cast<const uint4*>(L.meta)[((size_t)tile * C + c) * 64 + lane];
      const int cnt = __builtin_popcount(w.x) + __builtin_popcount(w.y) + __builtin_popcount(w.z) + __builtin_popcount(w.w);
      const uint32_t mis = (uint32_t)(nz_cur & 3);
      const uint32_t* s4 = reinterpret_cast<const uint32_t*>(L.dense + nz_cur - mis);
      const int nd = (cnt + (int)mis + 3) >> 2;
      for (int d = 0; d < nd; ++d) smem[slot_base / 4 + d] = s4[d];
      nz_cur += cnt;
      sb = slot_base + mis;
    } else {
      w = reinterpret_cast<const uint4*>(L.dense)[((size_t)tile * C + c) * 64 + lane];
      if constexpr (KIND == K_INT4_24) {
        const uint2 mv = reinterpret_cast<const uint2*>(L.meta)[((size_t)tile * C + c) * 64 + lane];
        mw = make_uint4(mv.x, mv.y, 0, 0);
      }
    }
    uint32_t wp[P];
    chunk_pairs<KIND>(w, mw, lanebase, sb, wp);
    if (n < N) {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int k = c * SPAN + 2 * j;
        const half2_t h = as_h2(wp[j]);
        _Float16 v0 = h.x, v1 = h.y;
        if (int_kind) {
          v0 = (_Float16)((float)h.x * scale);
          v1 = (_Float16)((float)h.y * scale);
        }
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

__global__ void debug_lowrank_kernel(const Layer L, float* L32, float* R32) {
  const int K = L.h.K, N = L.h.N, r = L.h.rank, g = L.h.group > 0 ? L.h.group : 1;
  const int half_r = (r + 1) / 2;
  const size_t nl = (size_t)K * r, nr = (size_t)r * N;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nl + nr; i += (size_t)gridDim.x * blockDim.x) {
    if (i < nl) {
      if (!L32) continue;
      const int k = (int)(i / r), j = (int)(i % r);
      float v;
      if (L.h.lr == CL_LR_INT4) {
        const int qv = (int)((L.L[(size_t)k * half_r + (j >> 1)] >> (4 * (j & 1))) & 0xF) - 8;
        v = (float)qv * (float)__builtin_bit_cast(_Float16, L.Lscale[(size_t)(k / g) * r + j]);
      } else {
        const uint16_t u = reinterpret_cast<const uint16_t*>(L.L)[i];
        v = L.h.lr == CL_LR_BF16 ? __uint_as_float((uint32_t)u << 16) : (float)__builtin_bit_cast(_Float16, u);
      }
      L32[i] = v;
    } else {
      if (!R32) continue;
      const size_t ii = i - nl;
      const int j = (int)(ii / N), n = (int)(ii % N);
      float v;
      if (L.h.lr == CL_LR_INT4) {
        const int qv = (int)((L.R[(size_t)j * (L.Npad / 2) + n / 2] >> (4 * (n & 1))) & 0xF) - 8;
        v = (float)qv * (float)__builtin_bit_cast(_Float16, L.Rscale[(size_t)(j / g) * L.Npad + n]);
      } else {
        const uint16_t u = reinterpret_cast<const uint16_t*>(L.R)[(size_t)j * L.Npad + n];
        v = L.h.lr == CL_LR_BF16 ? __uint_as_float((uint32_t)u << 16) : (float)__builtin_bit_cast(_Float16, u);
      }
      R32[ii] = v;
    }
  }
}

hipError_t launch_debug(const Layer& L, uint16_t* D16, uint16_t* S16, float* L32, float* R32, hipStream_t stream) {
  const cl_blob_header& h = L.h;
  const int cblk = 64;
  dim3 grid(h.n_tiles, (unsigned)ceil_div(h.chunks, cblk));
  dim3 grid1(h.n_tiles, 1);
  switch (h.dense) {
    case CL_DENSE_LUT3: hipLaunchKernelGGL(debug_dense_kernel<K_LUT3>, grid, dim3(64), 0, stream, L, D16, cblk); break;
    case CL_DENSE_LUT4: hipLaunchKernelGGL(debug_dense_kernel<K_LUT4>, grid, dim3(64), 0, stream, L, D16, cblk); break;
    case CL_DENSE_INT4:
      if (h.mask == CL_MASK_2_4)
        hipLaunchKernelGGL(debug_dense_kernel<K_INT4_24>, grid, dim3(64), 0, stream, L, D16, cblk);
      else
        hipLaunchKernelGGL(debug_dense_kernel<K_INT4>, grid, dim3(64), 0, stream, L, D16, cblk);
      break;
    default:
      if (h.mask == CL_MASK_BITMAP)
        hipLaunchKernelGGL(debug_dense_kernel<K_INT8_BM>, grid1, dim3(64), 0, stream, L, D16, cblk);
      else
        hipLaunchKernelGGL(debug_dense_kernel<K_INT8>, grid, dim3(64), 0, stream, L, D16, cblk);
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
