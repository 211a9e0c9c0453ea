// prefill_impl.h -- large-M forward on the matrix cores.
//
// y[M, N] = x'[M, K] . W^T on bf16 (bf16 activations) or fp16 (fp16
// activations) MFMA with fp32 accumulation, v_mfma_f32_32x32x16.  A workgroup
// owns a 128 x 128 output tile (128 activation rows m, 128 weight rows n) and
// has two roles of four wavefronts each:
//   - MFMA waves: each owns a 64 x 64 quarter (2 x 2 MFMA blocks) and only
//     reads operands from LDS and issues MFMAs;
//   - staging waves: load the activations and packed codes three K steps
//     ahead into a ring of register stages, dequantise the weight tile into
//     LDS through the same unpack functions as the decode path (two threads
//     per weight row), and add the step's outliers.
// Two LDS tile buffers: while the MFMA waves consume step s from one, the
// staging waves fill the other with step s + 1; two barriers per step (the
// outliers are added after the dequantised tile has landed).
//
// Outliers ("SqueezeLLM: Dense-and-Sparse Quantization", Approach: W = D + S)
// come as per-(tile, step) lists built when the layer is created: one entry
// per thread per step, added to the tile with LDS packed atomic adds.
//
// The rank-r correction ("SLiM" page, review highlights: y += (x' L) R) runs
// as extra K steps: the activation side is t = x' L split into t_hi + t_lo
// (two 16-bit numbers carrying t to about 16 significant bits), the weight side
// is R^T twice, so the MFMA adds t_hi R + t_lo R.  t is computed beforehand by
// this same kernel with L^T as the weight tile, split along K into partial
// sums that a small kernel adds in a fixed order.
//
// Weights enter the matrix cores as 16-bit values of the activation type: fp16
// LUT values exactly for fp16 activations, rounded to nearest-even bf16 for
// bf16 activations; integer codes times the row scale rounded to the type.
#pragma once
#include <hip/hip_runtime.h>

#include "layer.h"
#include "unpack.h"

namespace cl {

// Weight source of the prologue t = x' L: 16-bit L^T rows prepared at create.
enum { K_DENSE16 = 16 };

typedef __bf16 pf_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 pf_f16x8 __attribute__((ext_vector_type(8)));
typedef float pf_f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 pf_bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 pf_f16x2 __attribute__((ext_vector_type(2)));

constexpr int kPfBM = 128, kPfBN = kPfTileN, kPfThreads = 256;  // threads of one role
constexpr int kPfMaxSplit = 8;      // K splits of the prologue (the workspace holds this many partials)
constexpr int kPfMaxSteps = 1536;   // K steps whose outlier offsets fit the LDS cache
constexpr uint32_t kPfNoEntry = 0xFFFFFFFFu;

// Per weight kind: span of a chunk, K per step (a whole number of chunks and
// of 16), chunks each thread dequantises per step (two threads per row).
template <int KIND>
struct PfCfg {
  static constexpr int span = KIND == K_LUT3 ? 40 : KIND == K_INT4_24 ? 64 : KIND == K_INT8 ? 16 : 32;
  static constexpr int bk = KIND == K_LUT3 ? 80 : KIND == K_INT4_24 ? 128 : 64;
  static constexpr int cpt = bk / span / 2;  // chunks per thread per step
  static constexpr int vpt = bk / 2;         // weight values per thread per step
  static constexpr int ts = bk * 2 + 16;     // LDS bytes per tile row (padded: conflict-free 128-bit reads)
  static constexpr int tab = KIND == K_LUT3 ? 2 * 64 * 256 : KIND == K_LUT4 ? 2 * 16 * 256 : KIND == K_INT4_24 ? 256 : 0;
  static constexpr int buf = 2 * 128 * ts;   // one (A, B) tile pair
  static constexpr int cptr = tab + 2 * buf; // LDS cache of the workgroup's outlier offsets
  static constexpr int lds = cptr + (kPfMaxSteps + 1) * 4;
};
static_assert(PfCfg<K_LUT3>::bk == 80 && PfCfg<K_INT4_24>::bk == 128 && PfCfg<K_LUT4>::bk == 64,
              "step sizes must match pf_step_k()");

struct PfArgs {
  const uint16_t* x;   // activations [M][ldx], zero past K up to ldx
  int ldx, M, K;
  int N;               // weight rows that exist
  int Npad;            // rows with storage (codes, tables)
  // packed weights
  const uint4* dense;
  const uint8_t* meta;
  const uint16_t* table;
  int chunks;
  // 16-bit weight rows of the prologue (L^T, [nb16][ldb16], MFMA type)
  const uint16_t* b16;
  int ldb16, nb16;
  // outliers per (tile, step): offsets [tiles][nsteps_dense + 1], entries
  const int32_t* cptr;
  const uint32_t* cent;
  // rank steps: activations t_hi | t_lo [M][lda2], weights R^T | R^T [Npad][ldr16]
  const uint16_t* a2;
  int lda2;
  const uint16_t* r16;
  int ldr16;
  // output (the prologue's split z writes its partial at y + z * ystride)
  float* y;
  int ldy, ncols;      // store columns n < ncols
  size_t ystride;
  int nsteps, nsteps_dense;
  int steps_per_split;
};

template <bool BF16>
__device__ __forceinline__ uint32_t to16(float f) {
  if constexpr (BF16) return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// q * s of an integer format in the MFMA type, rounded once to nearest-even:
// an fp16 multiply rounds the exact product; for bf16 the product is exact in
// fp32 (at most 8 + 11 significant bits) and is rounded from there (rounding
// it to fp16 first would round twice).
template <bool BF16>
__device__ __forceinline__ uint32_t scale_pair16(uint32_t qpair, half2_t rscale) {
  if constexpr (!BF16) return as_u32(as_h2(qpair) * rscale);
  const half2_t q = as_h2(qpair);
  return to16<true>((float)q.x * (float)rscale.x) | (to16<true>((float)q.y * (float)rscale.y) << 16);
}

__device__ __forceinline__ uint4 pf_lds128(const uint32_t* lds, uint32_t byte_addr) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(lds) + byte_addr);
}
__device__ __forceinline__ void pf_st128(uint32_t* lds, uint32_t byte_addr, uint4 v) {
  *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(lds) + byte_addr) = v;
}

typedef __bf16 pf_bf16x16 __attribute__((ext_vector_type(16)));
typedef _Float16 pf_f16x16 __attribute__((ext_vector_type(16)));
typedef uint32_t pf_u32x8 __attribute__((ext_vector_type(8)));

// 2:4 weights on the sparse-A instruction (v_smfmac_f32_32x32x32): w holds the
// eight kept values of lane (weight row l mod 32, half h) -- the kept pairs of
// four consecutive groups of four k -- and idx (bits 16 ABID ..) their 2-bit
// positions; the activation operand of lane half h' is x at 8h'..8h'+7 of
// lane half 0's 16 k (x0) and of lane half 1's (x1).  The output holds weight
// rows along the lane's registers and activation rows along the lanes.
template <bool BF16, int ABID>
__device__ __forceinline__ pf_f32x16 pf_smfmac(uint4 w, uint4 x0, uint4 x1, uint32_t idx, pf_f32x16 c) {
  const pf_u32x8 b = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  if constexpr (BF16)
    return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(pf_bf16x8, w), __builtin_bit_cast(pf_bf16x16, b), c,
                                                     (int)idx, 0, ABID);
  return __builtin_amdgcn_smfmac_f32_32x32x32_f16(__builtin_bit_cast(pf_f16x8, w), __builtin_bit_cast(pf_f16x16, b), c,
                                                  (int)idx, 0, ABID);
}

template <bool BF16>
__device__ __forceinline__ pf_f32x16 pf_mfma(uint4 a, uint4 b, pf_f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(pf_bf16x8, a), __builtin_bit_cast(pf_bf16x8, b), c,
                                                   0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(pf_f16x8, a), __builtin_bit_cast(pf_f16x8, b), c, 0, 0,
                                                0);
}

// Adds one outlier entry to the weight tile at byte offset `btile` (row in tile,
// k in step, fp16 value) with a packed atomic add on the dword holding it.
template <bool BF16, int TS>
__device__ __forceinline__ void pf_add_outlier(uint32_t* smem, uint32_t btile, uint32_t e) {
  const uint32_t row = e & 127u, kl = (e >> 7) & 127u;
  const uint32_t addr = btile + row * TS + (kl & ~1u) * 2u;
  const uint32_t v16 = to16<BF16>((float)__builtin_bit_cast(_Float16, (uint16_t)(e >> 16)));
  const uint32_t pk = (kl & 1u) ? (v16 << 16) : v16;
  void* p = reinterpret_cast<uint8_t*>(smem) + addr;
  if constexpr (BF16)
    __builtin_amdgcn_ds_atomic_fadd_v2bf16((__attribute__((address_space(3))) pf_bf16x2*)p,
                                           __builtin_bit_cast(pf_bf16x2, pk));
  else
    __builtin_amdgcn_ds_atomic_fadd_v2f16((__attribute__((address_space(3))) pf_f16x2*)p,
                                          __builtin_bit_cast(pf_f16x2, pk));
}

// SP: INT4 2:4 without outliers on the sparse-A instruction.  The staging
// waves write each weight row's step as its 64 kept values in the MFMA type
// and its 2-bit positions (no zeros), the MFMA waves take half as many steps,
// and the accumulators hold the output transposed (weight rows along the
// registers); the rank steps then run with the weights as the first operand.
template <int KIND, bool BF16, bool SP = false>
__global__ void __launch_bounds__(2 * kPfThreads, 1) prefill_kernel(PfArgs a) {
  using C = PfCfg<KIND>;
  constexpr int BK = C::bk, TS = C::ts, SPAN = C::span, BUF = C::buf;
  static_assert(!SP || (KIND == K_INT4_24 && BK == 128), "the sparse tile holds one 128-k step of 2:4 rows");
  // sparse tile row: 64 kept values (128 bytes), then for each of the two
  // chunks a position word per MFMA lane half (16 bytes); 144 = 16 * 9 keeps
  // 16-byte reads of consecutive rows on distinct banks
  constexpr int TSS = 144;
  constexpr bool CODES = KIND != K_DENSE16;
  constexpr bool LUT = KIND == K_LUT3 || KIND == K_LUT4;
  constexpr int A_OFF = C::tab, B_OFF = C::tab + 128 * TS;  // tile buffer b at + b * BUF
  constexpr int AU = 128 * (BK / 8) / kPfThreads;           // 16-byte activation units per thread per step
  constexpr int BU = CODES ? C::cpt : C::vpt / 8;           // 16-byte weight loads per thread per step
  __shared__ __attribute__((aligned(16))) uint32_t smem[C::lds / 4];  // the only LDS object: tables at address 0

  // Waves 0..3 read the tiles and run the MFMAs; waves 4..7 load, dequantise
  // and stage the next step into the other tile buffer.
  const int gwave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const bool stager = gwave >= 4;
  const int tid = (int)threadIdx.x & (kPfThreads - 1), wave = gwave & 3, lane = tid & 63;
  const int n0 = blockIdx.x * kPfBN, m0 = blockIdx.y * kPfBM;
  const int s0 = blockIdx.z * a.steps_per_split;
  const int s1 = min(s0 + a.steps_per_split, a.nsteps);
  const bool has_csr = CODES && a.cptr != nullptr;
  int32_t* s_cptr = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(smem) + C::cptr);

  // ---- per-workgroup tables: LUTs of the 128 rows (two stacked lane-interleaved
  // tables in the MFMA type, so a lookup yields the operand pair), the 2:4
  // selectors, and the outlier offsets of this row tile ----
  auto lut16 = [&](uint32_t h) -> uint32_t {
    return BF16 ? to16<true>((float)__builtin_bit_cast(_Float16, (uint16_t)h)) : h;
  };
  if constexpr (KIND == K_LUT3) {
    const int r = (int)threadIdx.x & 127, e0 = 16 * ((int)threadIdx.x >> 7), row = n0 + r;
    const uint4 lv = row < a.Npad ? reinterpret_cast<const uint4*>(a.table)[row] : make_uint4(0, 0, 0, 0);
    const uint32_t lw[4] = {lv.x, lv.y, lv.z, lv.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = e0 + i, ca = e & 7, cb = e >> 3;
      const uint32_t va = lut16((lw[ca >> 1] >> (16 * (ca & 1))) & 0xFFFFu);
      const uint32_t vb = lut16((lw[cb >> 1] >> (16 * (cb & 1))) & 0xFFFFu);
      smem[((r >> 6) * 64 + e) * 64 + (r & 63)] = va | (vb << 16);
    }
  } else if constexpr (KIND == K_LUT4) {
    const int r = (int)threadIdx.x & 127, c0 = 4 * ((int)threadIdx.x >> 7), row = n0 + r;
    const uint2 lv = row < a.Npad ? reinterpret_cast<const uint2*>(a.table)[(size_t)row * 4 + (c0 >> 2)] : make_uint2(0, 0);
    const uint32_t lw[2] = {lv.x, lv.y};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      smem[((r >> 6) * 16 + c0 + i) * 64 + (r & 63)] = lut16((lw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
  } else if constexpr (KIND == K_INT4_24) {
    if (threadIdx.x < 16) {
      const uint2 e = seltab_2_4_entry((uint32_t)threadIdx.x);
      smem[2 * threadIdx.x] = e.x;
      smem[2 * threadIdx.x + 1] = e.y;
    }
  }
  if (has_csr) {
    const int32_t* cp = a.cptr + (size_t)blockIdx.x * (a.nsteps_dense + 1);
    for (int i = (int)threadIdx.x; i <= a.nsteps_dense; i += 2 * kPfThreads) s_cptr[i] = cp[i];
  }
  __syncthreads();

  if (stager) {
    // ---- staging waves ----
    // the weight row this thread dequantises and its half of each step
    const int nl = (wave & 1) * 64 + lane, half = wave >> 1, n = n0 + nl;
    const uint32_t lanebase = (uint32_t)lane * 4u, ebias = (uint32_t)(wave & 1) * (KIND == K_LUT3 ? 64u : 16u);
    // integer formats: the row scale multiplies every dequantised weight of the row
    half2_t rscale = {(_Float16)1.0f, (_Float16)1.0f};
    if constexpr (is_int_kind<KIND>()) {
      const _Float16 sc = n < a.Npad ? __builtin_bit_cast(_Float16, a.table[n]) : (_Float16)0.0f;
      rscale = half2_t{sc, sc};
    }
    // buffer resources: activation rows past M and weight rows past the
    // stored ones fall outside and read as zero
    const brsrc_t rx = make_rsrc(a.x, (uint32_t)a.M * (uint32_t)a.ldx * 2u);
    const brsrc_t rd = make_rsrc(CODES ? (const void*)a.dense : (const void*)a.b16,
                                 CODES ? (uint32_t)a.Npad * (uint32_t)a.chunks * 16u : (uint32_t)a.nb16 * (uint32_t)a.ldb16 * 2u);
    const brsrc_t rm = make_rsrc(a.meta, KIND == K_INT4_24 ? (uint32_t)a.Npad * (uint32_t)a.chunks * 8u : 0u);
    const brsrc_t rc = make_rsrc(a.cent, has_csr ? (uint32_t)s_cptr[a.nsteps_dense] * 4u : 0u);
    uint32_t xoff[AU];
#pragma unroll
    for (int i = 0; i < AU; ++i) {
      const int u = tid + i * kPfThreads, m = u / (BK / 8), kk = u - m * (BK / 8);
      xoff[i] = ((uint32_t)(m0 + m) * (uint32_t)a.ldx + 8u * kk) * 2u;
    }
    const uint32_t woff = CODES ? ((uint32_t)n * (uint32_t)a.chunks + (uint32_t)(half * C::cpt)) * 16u
                                : ((uint32_t)n * (uint32_t)a.ldb16 + (uint32_t)(half * C::vpt)) * 2u;

    // register stage of one step
    struct Stage {
      uint4 xa[AU];      // activation units
      uint4 wb[BU];      // code chunks, or 16-bit weights
      uint2 wm[C::cpt];  // 2:4 metadata
      uint32_t ce;       // this thread's outlier entry of the step (used when ce_ok)
      bool ce_ok;
    };
    // Every load of a step is issued whatever the step (a step past the dense
    // ones, or units past the activation row, read through a poisoned offset
    // that lands outside the buffer and returns zero): a fixed number of loads
    // per step lets the compiler wait for exactly the stage it consumes while
    // the two younger stages stay in flight.
    auto load_step = [&](Stage& st, int s, bool valid) {
      // activations: everything below ldx is x' or the zero padding past K
#pragma unroll
      for (int i = 0; i < AU; ++i) {
        const int kk8 = 8 * ((tid + i * kPfThreads) % (BK / 8));
        const bool ok = valid && s * BK + kk8 < a.ldx;
        st.xa[i] = bload128(rx, ok ? xoff[i] + (uint32_t)(s * BK * 2) : kNoLoad, 0);
      }
      if constexpr (CODES) {
        // chunks past a row's end only meet zero activations
        const uint32_t so = (uint32_t)(s * (BK / SPAN)) * 16u;
#pragma unroll
        for (int q = 0; q < C::cpt; ++q) {
          st.wb[q] = bload128(rd, valid ? woff + 16u * q + so : kNoLoad, 0);
          if constexpr (KIND == K_INT4_24)
            st.wm[q] = bload64(rm, valid ? (woff + 16u * q + so) >> 1 : kNoLoad, 0);
          else
            st.wm[q] = make_uint2(0, 0);
        }
        const int sc = valid ? s : 0;
        const int e0 = s_cptr[sc], cnt = s_cptr[sc + 1] - e0;
        const bool has = has_csr && valid && tid < cnt;
        st.ce = bload32(rc, has ? (uint32_t)(e0 + tid) * 4u : kNoLoad, 0);  // consumed three steps later
        st.ce_ok = has;
      } else {
        const int klo = s * BK + half * C::vpt;
#pragma unroll
        for (int j = 0; j < BU; ++j)
          st.wb[j] = bload128(rd, valid && klo + 8 * j < a.ldb16 ? woff + 16u * j + (uint32_t)(s * BK * 2) : kNoLoad, 0);
      }
    };
    // dense step s from stage st into tile buffer buf
    auto stage_dense = [&](const Stage& st, int s, int buf) {
      const uint32_t bo = (uint32_t)(buf * BUF);
#pragma unroll
      for (int i = 0; i < AU; ++i) {
        const int u = tid + i * kPfThreads, m = u / (BK / 8), kk = u - m * (BK / 8);
        pf_st128(smem, bo + (uint32_t)(A_OFF + m * TS + kk * 16), st.xa[i]);
      }
      const uint32_t brow = bo + (uint32_t)(B_OFF + nl * TS + half * C::vpt * 2);
      if constexpr (SP) {
        // this thread's chunk (64 k): word i holds the kept pairs of groups
        // 4i..4i+3, meta word j the positions of groups 8j..8j+7; position
        // words regrouped so that MFMA lane half h finds its bits of both of
        // the chunk's 32-k steps in one word (ABID 0 and 1)
        const uint32_t srow = bo + (uint32_t)(B_OFF + nl * TSS);
        const uint32_t ww[4] = {st.wb[0].x, st.wb[0].y, st.wb[0].z, st.wb[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t v[4];
          int4_word(ww[i], v);
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = scale_pair16<BF16>(v[j], rscale);
          pf_st128(smem, srow + (uint32_t)(half * 64 + 16 * i), make_uint4(v[0], v[1], v[2], v[3]));
        }
        const uint32_t m0w = st.wm[0].x, m1w = st.wm[0].y;
        *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(smem) + srow + 128u + (uint32_t)(half * 8)) =
            make_uint2((m0w & 0xFFFFu) | (m1w << 16), (m0w >> 16) | (m1w & 0xFFFF0000u));
      } else if constexpr (CODES) {
#pragma unroll
        for (int q = 0; q < C::cpt; ++q) {
          uint32_t wp[KindTraits<KIND>::pairs];
          chunk_pairs<KIND, false>(smem, st.wb[q], make_uint4(st.wm[q].x, st.wm[q].y, 0, 0), lanebase, 0u, wp, ebias);
          if constexpr (!LUT) {  // LUT tables already hold the MFMA type
#pragma unroll
            for (int j = 0; j < KindTraits<KIND>::pairs; ++j) wp[j] = scale_pair16<BF16>(wp[j], rscale);
          }
#pragma unroll
          for (int j = 0; j < KindTraits<KIND>::pairs / 4; ++j)
            pf_st128(smem, brow + (uint32_t)(q * SPAN * 2 + j * 16),
                     make_uint4(wp[4 * j], wp[4 * j + 1], wp[4 * j + 2], wp[4 * j + 3]));
        }
      } else {
#pragma unroll
        for (int j = 0; j < BU; ++j) pf_st128(smem, brow + (uint32_t)(j * 16), st.wb[j]);
      }
    };
    // outliers of dense step s, after the dequantised tile has landed
    auto add_outliers = [&](const Stage& st, int s, int buf) {
      if (!has_csr) return;
      const uint32_t btile = (uint32_t)(buf * BUF + B_OFF);
      if (st.ce_ok) pf_add_outlier<BF16, TS>(smem, btile, st.ce);
      const int e0 = s_cptr[s], cnt = s_cptr[s + 1] - e0;
      for (int i = kPfThreads + tid; i < cnt; i += kPfThreads) pf_add_outlier<BF16, TS>(smem, btile, a.cent[e0 + i]);
    };
    // rank step s: activations t_hi | t_lo and weights R^T | R^T, loaded directly
    auto stage_rank = [&](int s, int buf) {
      const uint32_t bo = (uint32_t)(buf * BUF);
      const int k0 = (s - a.nsteps_dense) * BK;
      const brsrc_t ra = make_rsrc(a.a2, (uint32_t)a.M * (uint32_t)a.lda2 * 2u);
      const brsrc_t rr = make_rsrc(a.r16, (uint32_t)a.Npad * (uint32_t)a.ldr16 * 2u);
      uint4 va[AU], vb[C::vpt / 8];
#pragma unroll
      for (int i = 0; i < AU; ++i) {
        const int u = tid + i * kPfThreads, m = u / (BK / 8), kk = u - m * (BK / 8);
        va[i] = k0 + 8 * kk < a.lda2 ? bload128(ra, ((uint32_t)(m0 + m) * (uint32_t)a.lda2 + (uint32_t)(k0 + 8 * kk)) * 2u, 0)
                                     : make_uint4(0, 0, 0, 0);
      }
      const int klo = k0 + half * C::vpt;
#pragma unroll
      for (int j = 0; j < C::vpt / 8; ++j)
        vb[j] = klo + 8 * j < a.ldr16 ? bload128(rr, ((uint32_t)n * (uint32_t)a.ldr16 + (uint32_t)(klo + 8 * j)) * 2u, 0)
                                      : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < AU; ++i) {
        const int u = tid + i * kPfThreads, m = u / (BK / 8), kk = u - m * (BK / 8);
        pf_st128(smem, bo + (uint32_t)(A_OFF + m * TS + kk * 16), va[i]);
      }
      const uint32_t brow = bo + (uint32_t)(B_OFF + nl * TS + half * C::vpt * 2);
#pragma unroll
      for (int j = 0; j < C::vpt / 8; ++j) pf_st128(smem, brow + (uint32_t)(j * 16), vb[j]);
    };

    // Three register stages in a ring, each loaded three steps before it is
    // staged.  Step t goes into tile buffer (t - s0) mod 2.  Per step: stage
    // the tile, barrier, add the outliers, refill the stage, barrier -- two
    // barriers per step like the MFMA waves, plus two after the last step.
    const int sd = max(s0, min(s1, a.nsteps_dense));  // dense steps [s0, sd), rank steps [sd, s1)
    Stage S0, S1, S2;
    load_step(S0, s0, s0 < sd);
    load_step(S1, s0 + 1, s0 + 1 < sd);
    load_step(S2, s0 + 2, s0 + 2 < sd);
    auto dense_step = [&](Stage& st, int t) {
      const int buf = (t - s0) & 1;
      stage_dense(st, t, buf);
      __syncthreads();
      add_outliers(st, t, buf);
      load_step(st, t + 3, t + 3 < sd);
      __syncthreads();
    };
    int t = s0;
    for (; t + 3 <= sd; t += 3) {
      dense_step(S0, t);
      dense_step(S1, t + 1);
      dense_step(S2, t + 2);
    }
    if (t < sd) dense_step(S0, t++);
    if (t < sd) dense_step(S1, t++);
    for (; t < s1; ++t) {
      stage_rank(t, (t - s0) & 1);
      __syncthreads();
      __syncthreads();
    }
    __syncthreads();
    __syncthreads();
    return;
  }

  // ---- MFMA waves: two barriers per step, matching the staging waves ----
  const int wm_ = wave & 1, wn_ = wave >> 1;
  pf_f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const uint32_t arow = (uint32_t)(A_OFF + (wm_ * 64 + (lane & 31)) * TS + (lane >> 5) * 16);
  const uint32_t brow0 = (uint32_t)(B_OFF + (wn_ * 64 + (lane & 31)) * TS + (lane >> 5) * 16);
  auto mma = [&](int buf, int ks0, int ks1) {
    const uint32_t bo = (uint32_t)(buf * BUF);
#pragma unroll
    for (int ks = ks0; ks < ks1; ++ks) {
      const uint4 a0 = pf_lds128(smem, bo + arow + ks * 32), a1 = pf_lds128(smem, bo + arow + 32 * TS + ks * 32);
      const uint4 b0 = pf_lds128(smem, bo + brow0 + ks * 32), b1 = pf_lds128(smem, bo + brow0 + 32 * TS + ks * 32);
      acc[0][0] = pf_mfma<BF16>(a0, b0, acc[0][0]);
      acc[0][1] = pf_mfma<BF16>(a0, b1, acc[0][1]);
      acc[1][0] = pf_mfma<BF16>(a1, b0, acc[1][0]);
      acc[1][1] = pf_mfma<BF16>(a1, b1, acc[1][1]);
    }
  };
  // SP: acc[j][i] = weight block j x activation block i (transposed output)
  const uint32_t srow0 = (uint32_t)(B_OFF + (wn_ * 64 + (lane & 31)) * TSS + (lane >> 5) * 16);  // kept values
  const uint32_t prow0 = (uint32_t)(B_OFF + (wn_ * 64 + (lane & 31)) * TSS + 128 + (lane >> 5) * 4);  // position words
  const uint32_t xrow0 = (uint32_t)(A_OFF + (wm_ * 64 + (lane & 31)) * TS + (lane >> 5) * 16);  // activations
  auto smma = [&](int buf, int c) {  // the two 32-k steps of chunk c
    const uint32_t bo = (uint32_t)(buf * BUF);
    const uint32_t p0 = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(smem) + bo + prow0 + 8 * c);
    const uint32_t p1 =
        *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(smem) + bo + prow0 + 32 * TSS + 8 * c);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = 2 * c + u;
      const uint4 w0 = pf_lds128(smem, bo + srow0 + q * 32), w1 = pf_lds128(smem, bo + srow0 + 32 * TSS + q * 32);
      const uint4 x0a = pf_lds128(smem, bo + xrow0 + q * 64), x0b = pf_lds128(smem, bo + xrow0 + q * 64 + 32);
      const uint4 x1a = pf_lds128(smem, bo + xrow0 + 32 * TS + q * 64),
                  x1b = pf_lds128(smem, bo + xrow0 + 32 * TS + q * 64 + 32);
      if (u == 0) {
        acc[0][0] = pf_smfmac<BF16, 0>(w0, x0a, x0b, p0, acc[0][0]);
        acc[0][1] = pf_smfmac<BF16, 0>(w0, x1a, x1b, p0, acc[0][1]);
        acc[1][0] = pf_smfmac<BF16, 0>(w1, x0a, x0b, p1, acc[1][0]);
        acc[1][1] = pf_smfmac<BF16, 0>(w1, x1a, x1b, p1, acc[1][1]);
      } else {
        acc[0][0] = pf_smfmac<BF16, 1>(w0, x0a, x0b, p0, acc[0][0]);
        acc[0][1] = pf_smfmac<BF16, 1>(w0, x1a, x1b, p0, acc[0][1]);
        acc[1][0] = pf_smfmac<BF16, 1>(w1, x0a, x0b, p1, acc[1][0]);
        acc[1][1] = pf_smfmac<BF16, 1>(w1, x1a, x1b, p1, acc[1][1]);
      }
    }
  };
  auto mma_t = [&](int buf, int ks0, int ks1) {  // dense steps with the weights first (SP's rank steps)
    const uint32_t bo = (uint32_t)(buf * BUF);
#pragma unroll
    for (int ks = ks0; ks < ks1; ++ks) {
      const uint4 a0 = pf_lds128(smem, bo + arow + ks * 32), a1 = pf_lds128(smem, bo + arow + 32 * TS + ks * 32);
      const uint4 b0 = pf_lds128(smem, bo + brow0 + ks * 32), b1 = pf_lds128(smem, bo + brow0 + 32 * TS + ks * 32);
      acc[0][0] = pf_mfma<BF16>(b0, a0, acc[0][0]);
      acc[0][1] = pf_mfma<BF16>(b0, a1, acc[0][1]);
      acc[1][0] = pf_mfma<BF16>(b1, a0, acc[1][0]);
      acc[1][1] = pf_mfma<BF16>(b1, a1, acc[1][1]);
    }
  };
  const int sdm = max(s0, min(s1, a.nsteps_dense));  // the last weight step + 1 (rank steps after it)
  __syncthreads();  // first staged step: tile landed
  __syncthreads();  // its outliers added
  for (int s = s0; s < s1; ++s) {
    const int buf = (s - s0) & 1;
    if constexpr (SP) {
      if (s < sdm) smma(buf, 0);
      else mma_t(buf, 0, (BK / 16) / 2);
      __syncthreads();
      if (s < sdm) smma(buf, 1);
      else mma_t(buf, (BK / 16) / 2, BK / 16);
    } else {
      mma(buf, 0, (BK / 16) / 2);
      __syncthreads();
      mma(buf, (BK / 16) / 2, BK / 16);
    }
    __syncthreads();
  }

  // ---- store: lane l of block (i, j) holds column n = l mod 32, rows 8 (v/4) + 4 (l/32) + v mod 4 ----
  float* yz = a.y + (size_t)blockIdx.z * a.ystride;
  if constexpr (SP) {
    // acc[j][i]: lane l holds activation row m = l mod 32 of block i for
    // weight rows 8 (v/4) + 4 (l/32) + v mod 4 of block j
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = m0 + wm_ * 64 + i * 32 + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int nn = n0 + wn_ * 64 + j * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (m < a.M && nn < a.ncols) yz[(size_t)m * a.ldy + nn] = acc[j][i][v];
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int nn = n0 + wn_ * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm_ * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < a.M && nn < a.ncols) yz[(size_t)m * a.ldy + nn] = acc[i][j][v];
      }
    }
}

template <int KIND, bool BF16>
hipError_t launch_prefill_t(const PfArgs& a, hipStream_t st) {
  if (a.cptr && a.nsteps_dense > kPfMaxSteps) return hipErrorInvalidValue;
  const int z = (int)ceil_div(a.nsteps, a.steps_per_split);
  dim3 grid((unsigned)ceil_div(a.ncols, kPfBN), (unsigned)ceil_div(a.M, kPfBM), (unsigned)z);
  if constexpr (KIND == K_INT4_24) {
    if (a.cptr == nullptr) {  // no outliers: the sparse-A instruction takes the stored 2:4 form
      hipLaunchKernelGGL((prefill_kernel<KIND, BF16, true>), grid, dim3(2 * kPfThreads), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((prefill_kernel<KIND, BF16>), grid, dim3(2 * kPfThreads), 0, st, a);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_prefill_kind(const PfArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? launch_prefill_t<KIND, true>(a, st) : launch_prefill_t<KIND, false>(a, st);
}

}  // namespace cl
