// decode_impl.h -- the decode kernel template (included by decode_<kind>.hip).
#pragma once
// batch 1..32 forward: y = x' (D + S + (L R)^T)^T on the vector ALUs.
//
// Work decomposition (one launch per layer):
//   * A workgroup owns one 64-row tile and 1/split of its K range, and has
//     five wavefronts.  Waves 0-3 stream the dense part: each lane owns one
//     row, loads 16-byte chunks of it (the tile-interleaved layout makes every
//     wavefront load one contiguous 1 KiB block), dequantises through LDS
//     tables and multiplies with activations the whole wavefront shares (they
//     arrive in scalar registers through s_load).  Wave 4 runs, at the same
//     time, the outlier CSR part and the rank-r epilogue for the tile; its
//     dependent loads hide behind the dense stream.
//   * The workgroup sums its waves in a fixed order; split-K workgroups of a
//     tile write partial sums and the last one to finish (counter per tile)
//     adds them in split order and stores y.  No float atomics: y is bitwise
//     reproducible.
//   * Workgroup ids are remapped so that the split-K partners of a tile run on
//     the same XCD (hardware dispatch goes round-robin over the 8 XCDs) and
//     exchange partial sums through one L2.
//
// The outlier part is balanced by entries, not rows ("SqueezeLLM: Dense-and-
// Sparse Quantization", measured-effects table: a balanced sparse kernel
// instead of a standard CSR kernel): the tile's nonzeros (contiguous in CSR)
// are cut into equal pieces per split and per lane; runs that cross a lane
// boundary are combined afterwards in lane order.
#include <hip/hip_runtime.h>

#include "layer.h"
#include "unpack.h"

namespace cl {

struct DecodeArgs {
  const uint4* dense;
  const uint8_t* meta;
  const int32_t* nzstart;  // bitmap: [Npad][4*split] byte offset of each wave slice's first kept value
  const uint16_t* table;
  const int32_t* rowptr;
  const int32_t* col;
  const uint16_t* val;
  const uint8_t* R;
  const uint16_t* Rscale;
  const float* t;
  const void* x;
  float* y;
  float* part;
  uint32_t* counters;
  int K, N, M, ldx, chunks, span, split, G, Gpad, rank, group, lr_kind, Npad;
};

// ---------------------------------------------------------------------------
// activations
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// acc += w_pair . x_pair  (fp16 x: one v_dot2; bf16 x: two mixed-precision fma)
template <bool BF16>
__device__ __forceinline__ float mac2(uint32_t w, uint32_t xv, float acc) {
  if constexpr (!BF16) {
    return __builtin_amdgcn_fdot2(as_h2(w), as_h2(xv), acc, false);
  } else {
    const half2_t h = as_h2(w);
    acc = __builtin_fmaf((float)h.x, bf16lo(xv), acc);
    return __builtin_fmaf((float)h.y, bf16hi(xv), acc);
  }
}

// ---------------------------------------------------------------------------
// one chunk: dequantise, then multiply with MB activation rows
// ---------------------------------------------------------------------------
template <int KIND, int MB, bool BF16, bool TAIL>
__device__ __forceinline__ void chunk_mac(uint4 w, uint4 mw, const uint32_t* __restrict__ xc, int ldx2,
                                          int M, int kvalid, uint32_t lanebase, uint32_t slot_base,
                                          float (&acc)[MB]) {
  constexpr int P = KindTraits<KIND>::pairs;
  uint32_t wp[P];
  chunk_pairs<KIND>(w, mw, lanebase, slot_base, wp);
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const uint32_t* xr = xc + (m < M ? m : M - 1) * ldx2;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      if (!TAIL || 2 * j < kvalid) acc[m] = mac2<BF16>(wp[j], xr[j], acc[m]);
    }
  }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int MB>
struct SideLds {
  // offsets (dwords) of the side-wave arrays after the main area
  static constexpr int acc = 0;                 // float [MB][64]
  static constexpr int rp = acc + MB * 64;      // int [65]
  static constexpr int brow = rp + 68;          // int [128]
  static constexpr int bsum = brow + 128;       // float [128][MB]
  static constexpr int flag = bsum + 128 * MB;  // int
  static constexpr int total = flag + 4;
};

template <int KIND, int MB>
struct DecodeLds {
  static constexpr int tab = KindTraits<KIND>::tab_dwords;
  static constexpr int red = 4 * MB * 64;
  static constexpr int main = tab > red ? tab : red;
  static constexpr int side = main;
  static constexpr int total = main + SideLds<MB>::total;
};

template <bool BF16>
__device__ __forceinline__ float load_x(const void* x, int ldx, int m, int k) {
  const uint16_t v = static_cast<const uint16_t*>(x)[(size_t)m * ldx + k];
  if constexpr (BF16) return __uint_as_float((uint32_t)v << 16);
  return (float)__builtin_bit_cast(_Float16, v);
}

template <int KIND, int MB, bool BF16>
__global__ void __launch_bounds__(320) decode_kernel(DecodeArgs a) {
  using LdsT = DecodeLds<KIND, MB>;
  using SL = SideLds<MB>;
  __shared__ uint32_t smem[LdsT::total];  // the only LDS object: tables start at address 0
  float* side_acc = reinterpret_cast<float*>(smem + LdsT::side + SL::acc);
  int* s_rp = reinterpret_cast<int*>(smem + LdsT::side + SL::rp);
  int* s_brow = reinterpret_cast<int*>(smem + LdsT::side + SL::brow);
  float* s_bsum = reinterpret_cast<float*>(smem + LdsT::side + SL::bsum);
  int* s_flag = reinterpret_cast<int*>(smem + LdsT::side + SL::flag);

  const int b = blockIdx.x;
  const int logical = (b & 7) * (a.Gpad >> 3) + (b >> 3);
  if (logical >= a.G) return;
  const int tile = logical / a.split, s = logical % a.split;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = tile * 64 + lane;
  const uint32_t lanebase = (uint32_t)lane * 4u;

  // ---- phase 1: tables (waves 0-3), side accumulators (wave 4) ----
  if (wave < 4) build_tables<KIND>(smem, a.table, tile, tid, 256);
  if (wave == 4) {
#pragma unroll
    for (int m = 0; m < MB; ++m) side_acc[m * 64 + lane] = 0.f;
    if (a.rowptr) {
      s_rp[lane] = a.rowptr[min(tile * 64 + lane, a.N)];
      if (lane == 0) s_rp[64] = a.rowptr[min(tile * 64 + 64, a.N)];
    }
  }
  __syncthreads();

  float acc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = 0.f;

  if (wave < 4) {
    // ---- phase 2a: dense stream over this wave's chunk range ----
    const int nsl = 4 * a.split, q = s * 4 + wave;
    const int cb = (int)((long long)a.chunks * q / nsl), ce = (int)((long long)a.chunks * (q + 1) / nsl);
    constexpr int SPAN = KindTraits<KIND>::span;
    const uint4* dp = a.dense + (size_t)tile * a.chunks * 64 + lane;
    const uint32_t* xbase = static_cast<const uint32_t*>(a.x);
    const int ldx2 = a.ldx >> 1;
    const int tail_valid = a.K - (a.chunks - 1) * SPAN;  // valid k in the last chunk
    uint32_t slot_base = 0;
    long long nz_cur = 0;
    if constexpr (KIND == K_INT8_BM) {
      slot_base = (uint32_t)(kBmSelDwords + (wave * 64 + lane) * kBmSlot) * 4u;
      nz_cur = a.nzstart[(size_t)n * nsl + q];
    }
    constexpr int D = 4;
    uint4 A[D], Am[D];
    auto load_group = [&](uint4 (&B)[D], uint4 (&Bm)[D], int c0) {
#pragma unroll
      for (int i = 0; i < D; ++i) {
        if (c0 + i < ce) {
          if constexpr (KIND == K_INT8_BM) {
            B[i] = reinterpret_cast<const uint4*>(a.meta)[((size_t)tile * a.chunks + c0 + i) * 64 + lane];
          } else {
            B[i] = dp[(size_t)(c0 + i) * 64];
          }
          if constexpr (KIND == K_INT4_24) {
            const uint2 mv = reinterpret_cast<const uint2*>(a.meta)[((size_t)tile * a.chunks + c0 + i) * 64 + lane];
            Bm[i] = make_uint4(mv.x, mv.y, 0, 0);
          }
        }
      }
    };
    load_group(A, Am, cb);
    for (int c = cb; c < ce; c += D) {
      uint4 B[D], Bm[D];
      load_group(B, Bm, c + D);
#pragma unroll
      for (int i = 0; i < D; ++i) {
        const int cc = c + i;
        if (cc < ce) {
          const uint32_t* xc = xbase + (size_t)cc * (SPAN / 2);
          if constexpr (KIND == K_INT8_BM) {
            // stage this chunk's kept values (<= 128 bytes) into the lane's LDS slot
            const uint4 bm = A[i];
            const int cnt = __builtin_popcount(bm.x) + __builtin_popcount(bm.y) +
                            __builtin_popcount(bm.z) + __builtin_popcount(bm.w);
            const uint8_t* src = reinterpret_cast<const uint8_t*>(a.dense) + nz_cur;
            const uint32_t mis = (uint32_t)(nz_cur & 3);
            const uint32_t* s4 = reinterpret_cast<const uint32_t*>(src - mis);
            const int nd = (cnt + (int)mis + 3) >> 2;  // dwords to stage, <= 33
            for (int d = 0; d < nd; ++d) smem[slot_base / 4 + d] = s4[d];
            nz_cur += cnt;
            if (cc == a.chunks - 1 && tail_valid < SPAN)
              chunk_mac<KIND, MB, BF16, true>(bm, bm, xc, ldx2, a.M, tail_valid, lanebase, slot_base + mis, acc);
            else
              chunk_mac<KIND, MB, BF16, false>(bm, bm, xc, ldx2, a.M, SPAN, lanebase, slot_base + mis, acc);
          } else {
            if (cc == a.chunks - 1 && tail_valid < SPAN)
              chunk_mac<KIND, MB, BF16, true>(A[i], Am[i], xc, ldx2, a.M, tail_valid, lanebase, 0u, acc);
            else
              chunk_mac<KIND, MB, BF16, false>(A[i], Am[i], xc, ldx2, a.M, SPAN, lanebase, 0u, acc);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < D; ++i) {
        A[i] = B[i];
        Am[i] = Bm[i];
      }
    }
  } else {
    // ---- phase 2b: side wave: balanced CSR outliers, then the rank-r epilogue ----
    if (a.rowptr) {
      const long long E0 = s_rp[0], E1 = s_rp[64], tot = E1 - E0;
      const long long sb = E0 + tot * s / a.split, se = E0 + tot * (s + 1) / a.split;
      const long long lb = sb + (se - sb) * lane / 64, le = sb + (se - sb) * (lane + 1) / 64;
      int slot0 = -1, slot1 = -1;
      float sum0[MB], sum1[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) sum0[m] = sum1[m] = 0.f;
      if (lb < le) {
        // row of entry lb: the last r with s_rp[r] <= lb
        int lo = 0, hi = 63;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_rp[mid] <= lb) lo = mid; else hi = mid - 1;
        }
        int row = lo;
        long long e = lb;
        while (e < le) {
          while (s_rp[row + 1] <= e) ++row;  // skip empty rows
          const long long rend = min((long long)s_rp[row + 1], le);
          float sum[MB];
#pragma unroll
          for (int m = 0; m < MB; ++m) sum[m] = 0.f;
          for (long long p = e; p < rend; ++p) {
            const float v = (float)__builtin_bit_cast(_Float16, a.val[p]);
            const int c = a.col[p];
#pragma unroll
            for (int m = 0; m < MB; ++m)
              sum[m] = __builtin_fmaf(v, load_x<BF16>(a.x, a.ldx, m < a.M ? m : a.M - 1, c), sum[m]);
          }
          const bool first = (e == lb), last = (rend == le);
          if (first) {
            slot0 = row;
#pragma unroll
            for (int m = 0; m < MB; ++m) sum0[m] = sum[m];
          } else if (last) {
            slot1 = row;
#pragma unroll
            for (int m = 0; m < MB; ++m) sum1[m] = sum[m];
          } else {
#pragma unroll
            for (int m = 0; m < MB; ++m) side_acc[m * 64 + row] += sum[m];
          }
          e = rend;
          ++row;
        }
      }
      s_brow[2 * lane] = slot0;
      s_brow[2 * lane + 1] = slot1;
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        s_bsum[(2 * lane) * MB + m] = sum0[m];
        s_bsum[(2 * lane + 1) * MB + m] = sum1[m];
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();
      // boundary runs, in lane order; lane m owns component m
      if (lane < MB) {
        for (int i = 0; i < 128; ++i) {
          const int r = s_brow[i];
          if (r >= 0) side_acc[lane * 64 + r] += s_bsum[i * MB + lane];
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
    if (a.lr_kind != CL_LR_NONE) {
      const int jb = a.rank * s / a.split, je = a.rank * (s + 1) / a.split;
      float lr[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) lr[m] = 0.f;
      for (int j = jb; j < je; ++j) {
        float r;
        if (a.lr_kind == CL_LR_INT4) {
          const uint32_t byte = a.R[(size_t)j * (a.Npad >> 1) + (n >> 1)];
          const int qv = (int)((byte >> (4 * (n & 1))) & 0xFu) - 8;
          r = (float)qv * (float)__builtin_bit_cast(_Float16, a.Rscale[(size_t)(j / a.group) * a.Npad + n]);
        } else {
          const uint16_t v = reinterpret_cast<const uint16_t*>(a.R)[(size_t)j * a.Npad + n];
          r = a.lr_kind == CL_LR_BF16 ? __uint_as_float((uint32_t)v << 16) : (float)__builtin_bit_cast(_Float16, v);
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) lr[m] = __builtin_fmaf(a.t[(m < a.M ? m : a.M - 1) * a.rank + j], r, lr[m]);
      }
#pragma unroll
      for (int m = 0; m < MB; ++m) side_acc[m * 64 + lane] += lr[m];
    }
  }

  // ---- phase 3: sum the dense waves in order, scale, add the side part ----
  __syncthreads();  // every wave is done with the tables
  float* red = reinterpret_cast<float*>(smem);
  if (wave < 4) {
#pragma unroll
    for (int m = 0; m < MB; ++m) red[(wave * MB + m) * 64 + lane] = acc[m];
  }
  __syncthreads();
  const bool int_kind = KIND >= K_INT4;
  for (int i = tid; i < MB * 64; i += 320) {
    const int m = i >> 6, l = i & 63;
    float d = red[(0 * MB + m) * 64 + l] + red[(1 * MB + m) * 64 + l];
    d += red[(2 * MB + m) * 64 + l];
    d += red[(3 * MB + m) * 64 + l];
    if (int_kind) d *= (float)__builtin_bit_cast(_Float16, a.table[tile * 64 + l]);
    red[(0 * MB + m) * 64 + l] = d + side_acc[m * 64 + l];
  }
  __syncthreads();

  // ---- phase 4: store, or combine split-K partials (last workgroup of the tile) ----
  if (a.split == 1) {
    for (int i = tid; i < MB * 64; i += 320) {
      const int m = i >> 6, l = i & 63, row = tile * 64 + l;
      if (m < a.M && row < a.N) a.y[(size_t)m * a.N + row] = red[m * 64 + l];
    }
    return;
  }
  float* mypart = a.part + ((size_t)tile * a.split + s) * (kMaxDecodeM * 64);
  for (int i = tid; i < MB * 64; i += 320) mypart[i] = red[i];
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = atomicAdd(&a.counters[tile], 1u);
    *s_flag = (old == (uint32_t)(a.split - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!*s_flag) return;
  __threadfence();
  const float* tp = a.part + (size_t)tile * a.split * (kMaxDecodeM * 64);
  for (int i = tid; i < MB * 64; i += 320) {
    const int m = i >> 6, l = i & 63, row = tile * 64 + l;
    float v = 0.f;
    for (int q = 0; q < a.split; ++q) v += __builtin_nontemporal_load(tp + (size_t)q * (kMaxDecodeM * 64) + i);
    if (m < a.M && row < a.N) a.y[(size_t)m * a.N + row] = v;
  }
  if (tid == 0) a.counters[tile] = 0u;  // ready for the next forward on this stream
}

// ---------------------------------------------------------------------------
// launch (instantiated per kind in decode_<kind>.hip)
// ---------------------------------------------------------------------------
template <int KIND, int MB, bool BF16>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<KIND, MB, BF16>), dim3(a.Gpad), dim3(320), 0, st, a);
  return hipGetLastError();
}

template <int KIND, bool BF16>
static hipError_t launch_mb(const DecodeArgs& a, hipStream_t st) {
  if (a.M <= 1) return launch_t<KIND, 1, BF16>(a, st);
  if (a.M <= 4) return launch_t<KIND, 4, BF16>(a, st);
  if (a.M <= 8) return launch_t<KIND, 8, BF16>(a, st);
  if (a.M <= 16) return launch_t<KIND, 16, BF16>(a, st);
  return launch_t<KIND, 32, BF16>(a, st);
}

template <int KIND>
hipError_t launch_decode_kind(const DecodeArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? launch_mb<KIND, true>(a, st) : launch_mb<KIND, false>(a, st);
}

}  // namespace cl
