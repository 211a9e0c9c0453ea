// decode_impl.h -- the decode kernel template (included by decode_<kind>.hip).
#pragma once
// batched decode forward (M = 5..32): y = x' (D + S + (L R)^T)^T on the vector ALUs.
// One lane per output row; this is the kernel for batches where the vector-ALU
// work per weight (one fp16 pair product per activation row) dominates.
//
// Work decomposition (one launch per layer):
//   * A workgroup owns one 64-row tile and 1/split of its K range, and has
//     five wavefronts.  Waves 0-3 stream the dense part: each lane owns one
//     row, loads 16-byte chunks of it (a whole 128-byte line per lane every
//     eight chunks), dequantises through LDS
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
// Activations are read through the constant address space: the loads are
// uniform across the wavefront, and this tells the compiler that nothing in
// the kernel writes them, so they become scalar (s_load) loads into SGPRs.
typedef const __attribute__((address_space(4))) uint32_t* xptr_t;

template <int KIND, int MB, bool BF16, bool TAIL>
__device__ __forceinline__ void chunk_mac(const uint32_t* lds, uint4 w, uint4 mw, xptr_t xc, int ldx2,
                                          int M, int kvalid, uint32_t lanebase, uint32_t slot_base,
                                          float (&acc)[MB]) {
  constexpr int P = KindTraits<KIND>::pairs;
  uint32_t wp[P];
  chunk_pairs<KIND>(lds, w, mw, lanebase, slot_base, wp);
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const xptr_t xr = xc + (m < M ? m : M - 1) * ldx2;
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
  // wave index via readfirstlane: the compiler then knows every wave-derived
  // value (chunk range, activation addresses) is uniform and uses scalar loads
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n = tile * 64 + lane;
  const uint32_t lanebase = (uint32_t)lane * 4u;

  constexpr int SPAN = KindTraits<KIND>::span;
  constexpr int D = 4;  // chunks per prefetch group
  float acc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = 0.f;

  // dense waves: chunk range, and the first group of loads issued before the
  // table is built so that its latency overlaps the table's
  const int nsl = 4 * a.split, q = s * 4 + (wave < 4 ? wave : 0);
  const int cb = (int)((long long)a.chunks * q / nsl), ce = (int)((long long)a.chunks * (q + 1) / nsl);
  // this lane's row in the row-major streams (one 128-byte line per eight chunks)
  const uint4* dp = a.dense + (size_t)n * a.chunks;
  const uint4* mp4 = reinterpret_cast<const uint4*>(a.meta) + (size_t)n * a.chunks;
  const uint2* mp2 = reinterpret_cast<const uint2*>(a.meta) + (size_t)n * a.chunks;
  // Software pipeline, D chunks deep: every load is unconditional (indices past
  // the wave's range are clamped to its last chunk, which is then already in
  // cache), so the compiler can wait for exactly the group it consumes.
  auto load_group = [&](uint4 (&B)[D], uint4 (&Bm)[D], int c0) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int cc = min(c0 + i, ce - 1);
      if constexpr (KIND == K_INT8_BM) {
        B[i] = mp4[cc];
      } else {
        B[i] = dp[cc];
      }
      if constexpr (KIND == K_INT4_24) {
        const uint2 mv = mp2[cc];
        Bm[i] = make_uint4(mv.x, mv.y, 0, 0);
      } else {
        Bm[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  uint4 A[D], Am[D];
  const bool dense_work = wave < 4 && cb < ce;
  if (dense_work) load_group(A, Am, cb);

  // ---- phase 1: tables (waves 0-3), side accumulators (wave 4) ----
  if (wave < 4) {
    build_tables<KIND>(smem, a.table, tile, tid, 256);
  } else {
#pragma unroll
    for (int m = 0; m < MB; ++m) side_acc[m * 64 + lane] = 0.f;
    if (a.rowptr) {
      s_rp[lane] = a.rowptr[min(tile * 64 + lane, a.N)];
      if (lane == 0) s_rp[64] = a.rowptr[min(tile * 64 + 64, a.N)];
    }
  }
  __syncthreads();

  if (wave < 4) {
    // ---- phase 2a: dense stream over this wave's chunk range ----
    const xptr_t xbase = (xptr_t)(a.x);
    const int ldx2 = a.ldx >> 1;
    const int tail_valid = a.K - (a.chunks - 1) * SPAN;  // valid k in the last chunk
    uint32_t slot_base = 0;
    long long nz_cur = 0;
    if constexpr (KIND == K_INT8_BM) {
      slot_base = (uint32_t)(kBmSelDwords + (wave * 64 + lane) * kBmSlot) * 4u;
      nz_cur = a.nzstart[(size_t)n * nsl + q];
    }
    if (dense_work) {
      for (int c = cb; c < ce; c += D) {
        uint4 B[D], Bm[D];
        load_group(B, Bm, c + D);
#pragma unroll
        for (int i = 0; i < D; ++i) {
          const int cc = c + i;
          if (cc < ce) {
            const xptr_t xc = xbase + (size_t)cc * (SPAN / 2);
            uint32_t sb = 0u;
            if constexpr (KIND == K_INT8_BM) {
              // stage this chunk's kept values (<= 128 bytes) into the lane's LDS slot
              const uint4 bm = A[i];
              const int cnt = __builtin_popcount(bm.x) + __builtin_popcount(bm.y) +
                              __builtin_popcount(bm.z) + __builtin_popcount(bm.w);
              const uint8_t* src = reinterpret_cast<const uint8_t*>(a.dense) + nz_cur;
              const uint32_t mis = (uint32_t)(nz_cur & 3);
              const uint32_t* s4 = reinterpret_cast<const uint32_t*>(src - mis);
              const int nd = (cnt + (int)mis + 3) >> 2;  // dwords to stage, <= 33
              uint32_t stage[33];
#pragma unroll
              for (int d = 0; d < 33; ++d) stage[d] = d < nd ? s4[d] : 0u;
#pragma unroll
              for (int d = 0; d < 33; ++d) smem[slot_base / 4 + d] = stage[d];
              nz_cur += cnt;
              sb = slot_base + mis;
            }
            if (cc == a.chunks - 1 && tail_valid < SPAN)
              chunk_mac<KIND, MB, BF16, true>(smem, A[i], Am[i], xc, ldx2, a.M, tail_valid, lanebase, sb, acc);
            else
              chunk_mac<KIND, MB, BF16, false>(smem, A[i], Am[i], xc, ldx2, a.M, SPAN, lanebase, sb, acc);
          }
        }
#pragma unroll
        for (int i = 0; i < D; ++i) {
          A[i] = B[i];
          Am[i] = Bm[i];
        }
      }
    }
  } else {
    // ---- phase 2b: side wave: balanced CSR outliers, then the rank-r epilogue ----
    // Loads are issued in batches (all columns and values of a batch, then all
    // activation gathers) so that a batch costs two memory round trips.
    constexpr int CB = MB <= 1 ? 16 : MB <= 4 ? 8 : MB <= 8 ? 4 : 2;
    if (a.rowptr) {
      const long long E0 = s_rp[0], E1 = s_rp[64], tot = E1 - E0;
      const long long sb = E0 + tot * s / a.split, se = E0 + tot * (s + 1) / a.split;
      const long long lb = sb + (se - sb) * lane / 64, le = sb + (se - sb) * (lane + 1) / 64;
      int slot0 = -1, slot1 = -1;
      float sum0[MB], sum1[MB], run[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) sum0[m] = sum1[m] = run[m] = 0.f;
      if (lb < le) {
        // row of entry lb: the last r with s_rp[r] <= lb
        int lo = 0, hi = 63;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_rp[mid] <= lb) lo = mid; else hi = mid - 1;
        }
        int row = lo;
        bool first = true;
        // runs: the first one (may be shared with the previous lane) goes to
        // slot 0, the last one (may be shared with the next lane) to slot 1,
        // the ones in between belong to this lane alone
        auto flush = [&](bool last) {
          if (first) {
            slot0 = row;
#pragma unroll
            for (int m = 0; m < MB; ++m) sum0[m] = run[m];
            first = false;
          } else if (last) {
            slot1 = row;
#pragma unroll
            for (int m = 0; m < MB; ++m) sum1[m] = run[m];
          } else {
#pragma unroll
            for (int m = 0; m < MB; ++m) side_acc[m * 64 + row] += run[m];
          }
#pragma unroll
          for (int m = 0; m < MB; ++m) run[m] = 0.f;
        };
        for (long long e0 = lb; e0 < le; e0 += CB) {
          int cidx[CB];
          float v[CB];
#pragma unroll
          for (int i = 0; i < CB; ++i) {
            const long long p = min(e0 + i, le - 1);
            cidx[i] = a.col[p];
            v[i] = e0 + i < le ? (float)__builtin_bit_cast(_Float16, a.val[p]) : 0.f;
          }
          float xv[CB][MB];
#pragma unroll
          for (int i = 0; i < CB; ++i)
#pragma unroll
            for (int m = 0; m < MB; ++m) xv[i][m] = load_x<BF16>(a.x, a.ldx, m < a.M ? m : a.M - 1, cidx[i]);
#pragma unroll
          for (int i = 0; i < CB; ++i) {
            const long long p = e0 + i;
            if (p < le) {
              while (s_rp[row + 1] <= p) {
                flush(false);
                ++row;
              }
#pragma unroll
              for (int m = 0; m < MB; ++m) run[m] = __builtin_fmaf(v[i], xv[i][m], run[m]);
            }
          }
        }
        flush(true);
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
      // Boundary runs: lane r adds the runs of row r, in lane order.  Only the
      // lanes whose entry ranges meet row r's entries can hold one, and those
      // are found by inverting the even split of [sb, se) over the 64 lanes.
      {
        const int r = lane;
        const long long rs = max((long long)s_rp[r], sb), re = min((long long)s_rp[r + 1], se);
        if (rs < re) {
          auto lane_of = [&](long long e) {  // largest l with lb(l) <= e
            int lo = 0, hi = 63;
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (sb + (se - sb) * mid / 64 <= e) lo = mid; else hi = mid - 1;
            }
            return lo;
          };
          const int la = lane_of(rs), lz = lane_of(re - 1);
          float add[MB];
#pragma unroll
          for (int m = 0; m < MB; ++m) add[m] = 0.f;
          for (int l = la; l <= lz; ++l) {
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
              if (s_brow[2 * l + sl] == r) {
#pragma unroll
                for (int m = 0; m < MB; ++m) add[m] += s_bsum[(2 * l + sl) * MB + m];
              }
            }
          }
#pragma unroll
          for (int m = 0; m < MB; ++m) side_acc[m * 64 + r] += add[m];
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
    if (a.lr_kind != CL_LR_NONE) {
      // y[m, n] += sum_j t[m, j] R_hat[j, n] over this split's share of the ranks
      const int jb = a.rank * s / a.split, je = a.rank * (s + 1) / a.split;
      typedef const __attribute__((address_space(4))) float* tptr_t;
      const tptr_t tp = (tptr_t)(a.t);
      constexpr int JB = 16;
      float lr[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) lr[m] = 0.f;
      for (int j0 = jb; j0 < je; j0 += JB) {
        float rv[JB];
#pragma unroll
        for (int i = 0; i < JB; ++i) {
          const int j = min(j0 + i, je - 1);
          float r;
          if (a.lr_kind == CL_LR_INT4) {  // R^T codes [Npad][ceil(r/2)], scales [Npad][ceil(r/g)]
            const uint32_t byte = a.R[(size_t)n * ((a.rank + 1) >> 1) + (j >> 1)];
            const int qv = (int)((byte >> (4 * (j & 1))) & 0xFu) - 8;
            const int gr = (a.rank + a.group - 1) / a.group;
            r = (float)qv * (float)__builtin_bit_cast(_Float16, a.Rscale[(size_t)n * gr + j / a.group]);
          } else {  // R^T [Npad][r]
            const uint16_t u = reinterpret_cast<const uint16_t*>(a.R)[(size_t)n * a.rank + j];
            r = a.lr_kind == CL_LR_BF16 ? __uint_as_float((uint32_t)u << 16) : (float)__builtin_bit_cast(_Float16, u);
          }
          rv[i] = j0 + i < je ? r : 0.f;
        }
#pragma unroll
        for (int i = 0; i < JB; ++i) {
          const int j = min(j0 + i, je - 1);
#pragma unroll
          for (int m = 0; m < MB; ++m) lr[m] = __builtin_fmaf(tp[(m < a.M ? m : a.M - 1) * a.rank + j], rv[i], lr[m]);
        }
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
  constexpr bool int_kind = is_int_kind<KIND>();
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
  // Partial sums cross workgroups (possibly on different XCDs, whose L2s are
  // not coherent with each other) through device-scope atomic stores and loads,
  // which bypass the non-coherent caches for these addresses only; a full
  // __threadfence() would write back and invalidate the whole L2 instead.
  float* mypart = a.part + ((size_t)tile * a.split + s) * (kMaxDecodeM * 64);
  for (int i = tid; i < MB * 64; i += 320) store_dev(mypart + i, red[i]);
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = (old == (uint32_t)(a.split - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!*s_flag) return;
  const float* tp = a.part + (size_t)tile * a.split * (kMaxDecodeM * 64);
  for (int i = tid; i < MB * 64; i += 320) {
    const int m = i >> 6, l = i & 63, row = tile * 64 + l;
    float v = 0.f;
    for (int qq = 0; qq < a.split; ++qq) v += load_dev(tp + (size_t)qq * (kMaxDecodeM * 64) + i);
    if (m < a.M && row < a.N) a.y[(size_t)m * a.N + row] = v;
  }
  if (tid == 0) __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next forward
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
  if constexpr (KIND == K_INT8_BM) {  // the bitmap format runs every M here
    if (a.M <= 1) return launch_t<KIND, 1, BF16>(a, st);
    if (a.M <= 4) return launch_t<KIND, 4, BF16>(a, st);
  }
  if (a.M <= 8) return launch_t<KIND, 8, BF16>(a, st);
  if (a.M <= 16) return launch_t<KIND, 16, BF16>(a, st);
  return launch_t<KIND, 32, BF16>(a, st);
}

template <int KIND>
hipError_t launch_decode_kind(const DecodeArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? launch_mb<KIND, true>(a, st) : launch_mb<KIND, false>(a, st);
}

}  // namespace cl
