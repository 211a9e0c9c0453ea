// prefill_impl.h -- large-M forward on the matrix cores.
//
// y[M, N] = x'[M, K] . W^T on bf16 (bf16 activations) or fp16 (fp16
// activations) MFMA with fp32 accumulation, v_mfma_f32_32x32x16.  A workgroup
// of four wavefronts owns a 128 x 128 output tile (128 activation rows m,
// 128 weight rows n); each wavefront a 64 x 64 quarter, 2 x 2 MFMA blocks.
// Per K step the workgroup
//   - stages the activation tile x'[m0.., k0..k0+BK) in LDS,
//   - dequantises the weight tile W[n0.., k0..) into LDS through the same
//     unpack functions as the decode path (two threads per weight row, one
//     chunk each), adding the row's outliers that fall in the step
//     ("SqueezeLLM: Dense-and-Sparse Quantization", Approach: W = D + S),
//   - and runs BK/16 MFMA steps over the two tiles,
// with the next step's activations and codes already loaded into registers.
//
// The rank-r correction ("SLiM" page, review highlights: y += (x' L) R) runs
// as extra K steps of the same loop: the activation side is t = x' L split
// into t_hi + t_lo (two 16-bit numbers whose sum carries t to about 16
// significant bits), the weight side is R^T twice, so the MFMA adds
// t_hi R + t_lo R.  t itself is computed beforehand by this same kernel with
// L^T as the weight tile (the "dense" weight kinds below).
//
// Weights enter the matrix cores as 16-bit values of the activation type: fp16
// LUT values exactly for fp16 activations; rounded to nearest-even bf16 for
// bf16 activations; integer codes times the row scale rounded to the type.
#pragma once
#include <hip/hip_runtime.h>

#include "layer.h"
#include "unpack.h"

namespace cl {

// Weight sources of the prologue t = x' L: L^T rows, 16-bit, or int4 with group scales.
enum { K_DENSE16 = 16, K_DENSE_INT4 = 17 };

typedef __bf16 pf_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 pf_f16x8 __attribute__((ext_vector_type(8)));
typedef float pf_f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfBM = 128, kPfBN = 128, kPfThreads = 256;

// Per weight kind: span of a chunk, K per step (a whole number of chunks and
// of 16), chunks each thread dequantises per step (two threads per row).
template <int KIND>
struct PfCfg {
  static constexpr int span = KIND == K_LUT3 ? 40 : KIND == K_INT4_24 ? 64 : KIND == K_INT8 ? 16 : 32;
  static constexpr int bk = KIND == K_LUT3 ? 80 : KIND == K_INT4_24 ? 128 : 64;
  static constexpr int cpt = bk / span / 2;                 // chunks per thread per step
  static constexpr int vpt = bk / 2;                        // weight values per thread per step
  static constexpr int ts = bk * 2 + 16;                    // LDS bytes per tile row (padded)
  static constexpr int tab = KIND == K_LUT3 ? 2 * 64 * 256 : KIND == K_LUT4 ? 2 * 16 * 256 : KIND == K_INT4_24 ? 256 : 0;
  static constexpr int lds = tab + 2 * 128 * ts;
};

struct PfArgs {
  const uint16_t* x;   // activations [M][ldx], zero past K up to ldx
  int ldx, M, K;
  int N;               // weight rows that exist (outputs: N, or rank for the prologue)
  int Npad;            // rows with storage (codes, tables): a multiple of 64
  // packed weights
  const uint4* dense;
  const uint8_t* meta;
  const uint16_t* table;
  int chunks;
  // prologue weights: L^T [rank][K] 16-bit, or int4 codes [rank][ceil(K/2)] + scales [rank][ceil(K/g)]
  const uint16_t* b16;
  const uint8_t* b4;
  const uint16_t* b4s;
  int group;
  int b_bf16;          // b16 holds bf16 (else fp16)
  // outliers
  const int32_t* rowptr;
  const int32_t* col;
  const uint16_t* val;
  // rank-r extension
  const float* t;      // [M][ldt]
  int ldt, rank, rp, lr_kind;
  const uint8_t* R;    // R^T [Npad][rank] 16-bit, or int4 [Npad][ceil(rank/2)]
  const uint16_t* Rscale;
  int rgroup;
  // output
  float* y;
  int ldy, ncols;      // store columns n < ncols
  int nsteps, nsteps_dense;
};

template <bool BF16>
__device__ __forceinline__ uint32_t to16(float f) {
  if constexpr (BF16) return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
template <bool BF16>
__device__ __forceinline__ float from16(uint32_t u) {
  if constexpr (BF16) return __uint_as_float(u << 16);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)u);
}
// fp16 pair -> pair of the MFMA type
template <bool BF16>
__device__ __forceinline__ uint32_t pair_to16(uint32_t h) {
  if constexpr (!BF16) return h;
  const half2_t v = as_h2(h);
  return to16<true>((float)v.x) | (to16<true>((float)v.y) << 16);
}

__device__ __forceinline__ uint4 pf_lds128(const uint32_t* lds, uint32_t byte_addr) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(lds) + byte_addr);
}
__device__ __forceinline__ void pf_st128(uint32_t* lds, uint32_t byte_addr, uint4 v) {
  *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(lds) + byte_addr) = v;
}

template <bool BF16>
__device__ __forceinline__ pf_f32x16 pf_mfma(uint4 a, uint4 b, pf_f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(pf_bf16x8, a), __builtin_bit_cast(pf_bf16x8, b), c,
                                                   0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(pf_f16x8, a), __builtin_bit_cast(pf_f16x8, b), c, 0, 0,
                                                0);
}

template <int KIND, bool BF16>
__global__ void __launch_bounds__(kPfThreads) prefill_kernel(PfArgs a) {
  using C = PfCfg<KIND>;
  constexpr int BK = C::bk, TS = C::ts, SPAN = C::span;
  constexpr bool CODES = KIND != K_DENSE16 && KIND != K_DENSE_INT4;
  constexpr int A_OFF = C::tab, B_OFF = C::tab + 128 * TS;
  constexpr int AU = 128 * (BK / 8) / kPfThreads;  // 16-byte activation units per thread per step
  __shared__ __attribute__((aligned(16))) uint32_t smem[C::lds / 4];  // the only LDS object: tables at address 0

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n0 = blockIdx.x * kPfBN, m0 = blockIdx.y * kPfBM;
  // the weight row this thread dequantises and its half of each step
  const int nl = (wave & 1) * 64 + lane, half = wave >> 1, n = n0 + nl;
  const uint32_t lanebase = (uint32_t)lane * 4u, ebias = (uint32_t)(wave & 1) * (KIND == K_LUT3 ? 64u : 16u);

  // ---- LUT tables of the 128 rows (two stacked lane-interleaved tables) ----
  if constexpr (KIND == K_LUT3) {
    for (int i = tid; i < 2 * 64 * 64; i += kPfThreads) {
      const int g = i >> 12, e = (i >> 6) & 63, l = i & 63, row = n0 + g * 64 + l;
      uint32_t v = 0;
      if (row < a.Npad) {
        const uint16_t* lt = a.table + (size_t)row * 8;
        v = (uint32_t)lt[e & 7] | ((uint32_t)lt[e >> 3] << 16);
      }
      smem[(g * 64 + e) * 64 + l] = v;
    }
  } else if constexpr (KIND == K_LUT4) {
    for (int i = tid; i < 2 * 16 * 64; i += kPfThreads) {
      const int g = i >> 10, c = (i >> 6) & 15, l = i & 63, row = n0 + g * 64 + l;
      smem[(g * 16 + c) * 64 + l] = row < a.Npad ? a.table[(size_t)row * 16 + c] : 0u;
    }
  } else if constexpr (KIND == K_INT4_24) {
    if (tid < 16) {
      const uint2 e = seltab_2_4_entry((uint32_t)tid);
      smem[2 * tid] = e.x;
      smem[2 * tid + 1] = e.y;
    }
  }
  // integer formats: the row scale multiplies every dequantised weight of the row
  half2_t rscale = {(_Float16)1.0f, (_Float16)1.0f};
  if constexpr (is_int_kind<KIND>()) {
    const _Float16 s = n < a.Npad ? __builtin_bit_cast(_Float16, a.table[n]) : (_Float16)0.0f;
    rscale = half2_t{s, s};
  }

  // ---- outlier cursor of row n: the next four entries in column order ----
  const bool has_csr = CODES && a.rowptr != nullptr;
  int cp = 0, ce = 0, bcol[4];
  float bval[4];
  if (has_csr) {
    cp = n < a.N ? a.rowptr[n] : 0;
    ce = n < a.N ? a.rowptr[n + 1] : 0;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = cp + i < ce;
    bcol[i] = ok ? a.col[cp + i] : 0x7FFFFFFF;
    bval[i] = ok ? (float)__builtin_bit_cast(_Float16, a.val[cp + i]) : 0.f;
  }

  // ---- register stages of one step ----
  uint4 xa[AU];        // activation units
  uint4 wc[C::cpt];    // code chunks
  uint2 wm[C::cpt];    // 2:4 metadata
  auto load_step = [&](int s) {
    // activations (dense steps only; the rank steps build theirs directly)
#pragma unroll
    for (int i = 0; i < AU; ++i) {
      const int u = tid + i * kPfThreads, m = u / (BK / 8), kk = u - m * (BK / 8);
      const int k = s * BK + 8 * kk;
      const bool ok = s < a.nsteps_dense && m0 + m < a.M && k < a.ldx;
      xa[i] = ok ? *reinterpret_cast<const uint4*>(a.x + (size_t)(m0 + m) * a.ldx + k) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (CODES) {
#pragma unroll
      for (int q = 0; q < C::cpt; ++q) {
        const int c = s * (BK / SPAN) + half * C::cpt + q;
        const bool ok = s < a.nsteps_dense && c < a.chunks && n < a.Npad;
        const size_t idx = (size_t)n * a.chunks + c;
        wc[q] = ok ? a.dense[idx] : make_uint4(0, 0, 0, 0);
        if constexpr (KIND == K_INT4_24)
          wm[q] = ok ? reinterpret_cast<const uint2*>(a.meta)[idx] : make_uint2(0, 0);
        else
          wm[q] = make_uint2(0, 0);
      }
    }
  };

  // 16-bit weight of the prologue source at (row n, k), as float
  auto dense_w = [&](int k) -> float {
    if (n >= a.N || k >= a.K) return 0.f;
    if constexpr (KIND == K_DENSE16) {
      const uint32_t u = a.b16[(size_t)n * a.K + k];
      return a.b_bf16 ? __uint_as_float(u << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)u);
    } else {
      const uint32_t byte = a.b4[(size_t)n * ((a.K + 1) >> 1) + (k >> 1)];
      const int q = (int)((byte >> (4 * (k & 1))) & 0xFu) - 8;
      const int ng = (a.K + a.group - 1) / a.group;
      return (float)q * (float)__builtin_bit_cast(_Float16, a.b4s[(size_t)n * ng + k / a.group]);
    }
  };
  // rank-r factor R^T at (row n, j), as float
  auto r_w = [&](int j) -> float {
    if (n >= a.N || j >= a.rank) return 0.f;
    if (a.lr_kind == CL_LR_INT4) {
      const uint32_t byte = a.R[(size_t)n * ((a.rank + 1) >> 1) + (j >> 1)];
      const int q = (int)((byte >> (4 * (j & 1))) & 0xFu) - 8;
      const int ng = (a.rank + a.rgroup - 1) / a.rgroup;
      return (float)q * (float)__builtin_bit_cast(_Float16, a.Rscale[(size_t)n * ng + j / a.rgroup]);
    }
    const uint32_t u = reinterpret_cast<const uint16_t*>(a.R)[(size_t)n * a.rank + j];
    return a.lr_kind == CL_LR_BF16 ? __uint_as_float(u << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)u);
  };

  // ---- write step s into the LDS tiles ----
  auto stage_step = [&](int s) {
    if (s < a.nsteps_dense) {
#pragma unroll
      for (int i = 0; i < AU; ++i) {
        const int u = tid + i * kPfThreads, m = u / (BK / 8), kk = u - m * (BK / 8);
        pf_st128(smem, (uint32_t)(A_OFF + m * TS + kk * 16), xa[i]);
      }
    } else {
      // rank steps: virtual index v < rp -> t_hi[m][v], rp <= v < 2 rp -> t_lo[m][v - rp]
#pragma unroll
      for (int i = 0; i < AU; ++i) {
        const int u = tid + i * kPfThreads, m = u / (BK / 8), kk = u - m * (BK / 8);
        const int v0 = (s - a.nsteps_dense) * BK + 8 * kk;
        const bool lo = v0 >= a.rp;
        const int j0 = lo ? v0 - a.rp : v0;
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j0 + e;
          const float tv = (m0 + m < a.M && v0 < 2 * a.rp && j < a.rank) ? a.t[(size_t)(m0 + m) * a.ldt + j] : 0.f;
          const uint32_t hi = to16<BF16>(tv);
          h[e] = lo ? to16<BF16>(tv - from16<BF16>(hi)) : hi;
        }
        pf_st128(smem, (uint32_t)(A_OFF + m * TS + kk * 16),
                 make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16));
      }
    }
    const uint32_t brow = (uint32_t)(B_OFF + nl * TS + half * C::vpt * 2);
    const int klo = s * BK + half * C::vpt;  // first k of this thread's part of the step
    if (s < a.nsteps_dense) {
      if constexpr (CODES) {
#pragma unroll
        for (int q = 0; q < C::cpt; ++q) {
          uint32_t wp[KindTraits<KIND>::pairs];
          chunk_pairs<KIND, false>(smem, wc[q], make_uint4(wm[q].x, wm[q].y, 0, 0), lanebase, 0u, wp, ebias);
#pragma unroll
          for (int j = 0; j < KindTraits<KIND>::pairs; ++j) {
            if constexpr (is_int_kind<KIND>()) wp[j] = as_u32(as_h2(wp[j]) * rscale);
            wp[j] = pair_to16<BF16>(wp[j]);
          }
#pragma unroll
          for (int j = 0; j < KindTraits<KIND>::pairs / 4; ++j)
            pf_st128(smem, brow + (uint32_t)(q * SPAN * 2 + j * 16),
                     make_uint4(wp[4 * j], wp[4 * j + 1], wp[4 * j + 2], wp[4 * j + 3]));
        }
        // outliers of row n inside [klo, klo + vpt): added to the tile entries
        if (has_csr) {
          const int khi = klo + C::vpt;
          while (bcol[0] < khi) {
            if (bcol[0] >= klo) {
              const uint32_t ad = brow + (uint32_t)(bcol[0] - klo) * 2u;
              const float w = from16<BF16>(lds_u16(smem, ad)) + bval[0];
              *reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(smem) + ad) = (uint16_t)to16<BF16>(w);
            }
            ++cp;
            bcol[0] = bcol[1];
            bcol[1] = bcol[2];
            bcol[2] = bcol[3];
            bval[0] = bval[1];
            bval[1] = bval[2];
            bval[2] = bval[3];
            const bool ok = cp + 3 < ce;
            bcol[3] = ok ? a.col[cp + 3] : 0x7FFFFFFF;
            bval[3] = ok ? (float)__builtin_bit_cast(_Float16, a.val[cp + 3]) : 0.f;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < C::vpt / 8; ++j) {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = to16<BF16>(dense_w(klo + 8 * j + e));
          pf_st128(smem, brow + (uint32_t)(j * 16),
                   make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16));
        }
      }
    } else {
      // rank steps: R^T row n at virtual index v -> j = v mod rp
      const int v0 = (s - a.nsteps_dense) * BK + half * C::vpt;
#pragma unroll
      for (int j = 0; j < C::vpt / 8; ++j) {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int v = v0 + 8 * j + e;
          const int jj = v < a.rp ? v : v - a.rp;
          h[e] = v < 2 * a.rp ? to16<BF16>(r_w(jj)) : 0u;
        }
        pf_st128(smem, brow + (uint32_t)(j * 16),
                 make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16));
      }
    }
  };

  // ---- main loop ----
  const int wm_ = wave & 1, wn_ = wave >> 1;
  pf_f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  __syncthreads();  // tables
  load_step(0);
  const uint32_t arow = (uint32_t)(A_OFF + (wm_ * 64 + (lane & 31)) * TS + (lane >> 5) * 16);
  const uint32_t bcol0 = (uint32_t)(B_OFF + (wn_ * 64 + (lane & 31)) * TS + (lane >> 5) * 16);
  for (int s = 0; s < a.nsteps; ++s) {
    stage_step(s);
    __syncthreads();
    if (s + 1 < a.nsteps) load_step(s + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const uint4 a0 = pf_lds128(smem, arow + ks * 32), a1 = pf_lds128(smem, arow + 32 * TS + ks * 32);
      const uint4 b0 = pf_lds128(smem, bcol0 + ks * 32), b1 = pf_lds128(smem, bcol0 + 32 * TS + ks * 32);
      acc[0][0] = pf_mfma<BF16>(a0, b0, acc[0][0]);
      acc[0][1] = pf_mfma<BF16>(a0, b1, acc[0][1]);
      acc[1][0] = pf_mfma<BF16>(a1, b0, acc[1][0]);
      acc[1][1] = pf_mfma<BF16>(a1, b1, acc[1][1]);
    }
    __syncthreads();
  }

  // ---- store: lane l of block (i, j) holds column n = l mod 32, rows 8 (v/4) + 4 (l/32) + v mod 4 ----
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int nn = n0 + wn_ * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm_ * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < a.M && nn < a.ncols) a.y[(size_t)m * a.ldy + nn] = acc[i][j][v];
      }
    }
}

template <int KIND, bool BF16>
hipError_t launch_prefill_t(const PfArgs& a, hipStream_t st) {
  dim3 grid((unsigned)ceil_div(a.ncols, kPfBN), (unsigned)ceil_div(a.M, kPfBM));
  hipLaunchKernelGGL((prefill_kernel<KIND, BF16>), grid, dim3(kPfThreads), 0, st, a);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_prefill_kind(const PfArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? launch_prefill_t<KIND, true>(a, st) : launch_prefill_t<KIND, false>(a, st);
}

}  // namespace cl
