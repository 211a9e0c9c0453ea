// decode_stream.h -- batch-1 forward: every wavefront streams an equal share of
// its workgroup's code chunks.
//
// A workgroup of up to 16 wavefronts owns a contiguous block of rows, sized so
// that every workgroup of the launch is resident at once.  The rows' code
// chunks are contiguous in memory (row-major, `chunks` per row), so the
// workgroup's chunks form one flat range; each wavefront takes an equal slice
// of it (whole passes of 64 chunks, at least one row's worth), whatever the
// row boundaries, and walks it one chunk per lane per pass.  No lane idles at
// the end of a row (K = 8192 in 40-weight chunks is 205 chunks: four 64-lane
// passes per row would leave 20% of the lanes without work), the code loads
// need no per-load address work, and the loads of the next passes are in
// flight while one pass is multiplied.
//
// A row has at least 64 chunks, so a pass meets at most one row boundary, at a
// lane that is the same for the whole wavefront: the lanes before it are in
// row n, the lanes from it on in row n + 1.  At that pass each lane's partial
// sum of row n goes to LDS; a row split between two slices gets one such
// vector from each.  After the walk, each row's partial vectors, its outliers
// (the balanced spread over the lanes of "SqueezeLLM: Dense-and-Sparse
// Quantization", Approach and measured-effects table) and its rank-r term
// ("SLiM" page, review highlights) are summed by one wavefront reduction.
// Everything besides the codes (activations, converted to fp16 with a row
// scale when they are bf16; LUT tables or row scales; row pointers; outliers;
// rank-factor rows) is staged in LDS once per workgroup before the walk, so
// the loads inside it are the code chunks alone and the compiler's load
// counting stays exact.  t = x' L_hat comes from the launch's first workgroups.
#pragma once
#include <hip/hip_runtime.h>

#include "decode_rows.h"

namespace cl {

constexpr int kStMaxWaves = 16;  // wavefronts per workgroup
constexpr int kStOutLoads = 6;   // outlier entries a thread stages
#ifndef CL_ST_NB
#define CL_ST_NB 4
#endif
#ifndef CL_ST_NBUF
#define CL_ST_NBUF 2
#endif
constexpr int kStNB = CL_ST_NB;      // passes per block of the code stream
constexpr int kStNBUF = CL_ST_NBUF;  // blocks in flight

struct StreamArgs {
  RowArgs r;            // pointers, sizes, activation edits, the in-launch prologue
  int rows_per_wg;      // rows of each workgroup (the last may have fewer)
  int lds_x;            // dynamic LDS byte offsets: activations,
  int lds_max;          //   per-wavefront maxima (bf16 rows),
  int lds_meta;         //   per-row LUT values / scales,
  int lds_rp;           //   row pointers (rows + 1),
  int lds_rank;         //   rank-factor rows (rows x rank_row_bytes),
  int lds_rsc;          //   int4 rank-factor scales (rows x rsc_row_bytes),
  int lds_part0;        //   per-lane partial sums: one vector per row,
  int lds_part1;        //   one per wavefront (its first row, when its slice starts inside it),
  int lds_out;          //   outliers: out_cap 16-bit columns, then out_cap fp16 values,
  int lds_t;            //   t = x' L_hat (rank floats)
  int rank_row_bytes;   // bytes of one R^T row (16-bit: 2 rank, int4: ceil(rank / 2))
  int rank_row_stride;  // its LDS stride: 16 bytes more when a power of two of at least 16
                        // (rows that a wavefront reads together then fall on different banks)
  int rsc_row_bytes;    // bytes of one row of int4 R^T scales
  int out_cap;          // outlier entries staged per workgroup (<= threads * kStOutLoads)
  int lr_readers;       // readers of t in a recorded launch (one per row workgroup)
  int lr_nl;            // int4 factors in 1024-thread prologue blocks: 16-byte loads a thread (1 or 4)
};

// Static LDS of the tables, the kernel's one static array (at LDS address 0, so
// that lookups at offsets built by v_perm need no base added): LUT row tables
// of up to 128 (LUT3, 256 bytes each) or 64 (LUT4, 1 KiB each) rows, or the
// 2:4 selector table.
template <int KIND>
constexpr int stream_tab_bytes() {
  return KIND == K_LUT3 ? 128 * 256 : KIND == K_LUT4 ? 64 * 1024 : KIND == K_INT4_24 ? 256 : 16;
}

// Chunks of one wavefront's slice: the workgroup's F chunks over wpg
// wavefronts, rounded up to whole passes, and at least one row (so that a row
// spans at most two slices).
__host__ __device__ inline int stream_slice(int F, int C, int wpg) {
  const int even = ((F + wpg - 1) / wpg + 63) & ~63, row = (C + 63) & ~63;
  return even > row ? even : row;
}

// Prologue blocks of a streaming launch: a workgroup of 16 wavefronts works on
// a K slice four (fp16 / bf16 factors) or one or four (int4, nl) times as long
// as the 256-thread block's.
inline int stream_lr_slices(int lr_S, int threads, int lr_mode, int nl = 1) {
  const int f = threads != 1024 ? 1
                : lr_mode == 0 ? lr_slice_rows<0, 1024>() / kLrSlice
                               : (nl == 4 ? lr_slice_rows<1, 1024, 4>() : lr_slice_rows<1, 1024>()) / kLrSlice;
  return (lr_S + f - 1) / f;
}

// 2:4 gather selector (16 entries, one per meta nibble i0 | i1 << 2): the
// bytes of activations i0 and i1 of a group of four, picked by v_perm from the
// group's two activation pairs.
__device__ __forceinline__ uint32_t xsel_2_4_entry(uint32_t nib) {
  const uint32_t i0 = nib & 3u, i1 = nib >> 2;
  return (2u * i0) | ((2u * i0 + 1u) << 8) | ((2u * i1) << 16) | ((2u * i1 + 1u) << 24);
}

// One 2:4 chunk (sixteen groups of four weights, two kept in each): the kept
// values as fp16 pairs qv[g] = (v0, v1) and the activations at their
// positions xg[g] = (x[i0], x[i1]), gathered from the chunk's activation pairs
// xv with the selector of the group's meta nibble (table at LDS address 0).
// Half the dot products of expanding the weights to four positions with zeros.
__device__ __forceinline__ void int4_24_gather(const uint32_t* lds, const uint4& w, const uint2& mw, const uint32_t (&xv)[32],
                                               uint32_t (&qv)[16], uint32_t (&xg)[16]) {
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  const uint32_t mm[2] = {mw.x, mw.y};
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    qv[g] = int4_pair(ww[g / 4], 4 * (g % 4));
    const uint32_t sel = lds_u32(lds, ((mm[g / 8] >> (4 * (g % 8))) & 0xFu) * 4u);
    xg[g] = perm(xv[2 * g + 1], xv[2 * g], sel);
  }
}

// XR = activation slots staged per thread, LR = low-rank part, EDIT = raw
// activations edited (clamp, per-channel factors) while staged.
template <int KIND, bool BF16, int XR, bool LR, bool EDIT>
__global__ void __launch_bounds__(1024) decode_stream_kernel(StreamArgs sa) {
  const RowArgs& a = sa.r;
  constexpr int NB = KIND == K_INT4_24 ? 2 : kStNB;  // 2:4 chunks dequantise to 32 pairs: fewer blocks in registers
  constexpr int SPAN = KindTraits<KIND>::span, P = KindTraits<KIND>::pairs, XD = SPAN / 8;
  constexpr int XS = RowX<KIND>::stride, XSL = RowX<KIND>::slots;
  constexpr bool LUT = KIND == K_LUT3 || KIND == K_LUT4;
  constexpr uint32_t RTB = (uint32_t)row_table_bytes<KIND>();
  constexpr int TB = KIND == K_LUT4 ? 32 : KIND == K_LUT3 ? 16 : 2;  // metadata bytes per row
  __shared__ __attribute__((aligned(16))) uint32_t stab[stream_tab_bytes<KIND>() / 4];  // at LDS address 0
  extern __shared__ __attribute__((aligned(16))) uint32_t sdyn[];
  uint8_t* sb = reinterpret_cast<uint8_t*>(sdyn);
  const int tid = threadIdx.x, nthr = blockDim.x, wpg = nthr >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  if constexpr (LR) {
    if ((int)blockIdx.x < a.lr_wgs) {  // a prologue workgroup
      const int b = blockIdx.x, S = a.lrp.S, s = b % S, tj = (b / S) % a.lr_ntj, tm = b / (S * a.lr_ntj);
      if (nthr == 1024) {
        if (a.lr_mode == 0) lr_split_block<0, 1, BF16, EDIT, 1024, true>(a.lrp, s, tj, tm, a.lr_ntj, sb);
        else if (sa.lr_nl == 4) lr_split_block<1, 1, BF16, EDIT, 1024, true, 4>(a.lrp, s, tj, tm, a.lr_ntj, sb);
        else lr_split_block<1, 1, BF16, EDIT, 1024, true>(a.lrp, s, tj, tm, a.lr_ntj, sb);
      } else {
        if (a.lr_mode == 0) lr_split_block<0, 1, BF16, EDIT, 256, true>(a.lrp, s, tj, tm, a.lr_ntj, sb);
        else lr_split_block<1, 1, BF16, EDIT, 256, true>(a.lrp, s, tj, tm, a.lr_ntj, sb);
      }
      return;
    }
  }
  const int wg = (int)blockIdx.x - (LR ? a.lr_wgs : 0);
  const int r0 = wg * sa.rows_per_wg;            // first row of the workgroup
  const int rw = min(sa.rows_per_wg, a.N - r0);  // its rows (>= 1)
  const int C = a.chunks, F = rw * C;            // chunks per row, of the workgroup
  const int Lw = stream_slice(F, C, wpg);
  const int f0 = wave * Lw, f1 = min(F, f0 + Lw);  // this wavefront's slice [f0, f1)
  const int np = f0 < f1 ? (f1 - f0 + 63) >> 6 : 0;
  const bool has_csr = a.rowptr != nullptr;
  // the workgroup's outliers [E0, E1): scalar loads, waited for with the activations
  const int E0 = has_csr ? a.rowptr[r0] : 0, E1 = has_csr ? a.rowptr[r0 + rw] : 0;

  // ---- activations and LUT values / scales, staged before the walk and
  // waited for before anything else is asked for ----
  const int SM = C * XSL;  // activation slots of the row
  const brsrc_t rx = make_rsrc(a.x, (uint32_t)a.ldx * 2u);
  auto x_src = [&](int s) -> uint32_t {  // byte offset of slot s in x (and in the factors), or kNoLoad
    int k, d = 0;
    if constexpr (XD == XSL) {
      k = 8 * s;  // no padding slots: slot s holds k = 8 s .. 8 s + 7
    } else {
      const int c = s / XSL;
      d = s - c * XSL;
      k = c * SPAN + 8 * d;
    }
    const bool ok = s < SM && d < XD && k < a.ldx;
    return ok ? (uint32_t)k * 2u : kNoLoad;
  };
  uint4 xs[XR];
#pragma unroll
  for (int i = 0; i < XR; ++i) xs[i] = bload128(rx, x_src(i * nthr + tid), 0);
  uint4 xf[EDIT ? XR : 1];
  if constexpr (EDIT) {
    const brsrc_t rf = make_rsrc(a.xscale, a.xscale ? (uint32_t)a.ldx * 2u : 0u);
#pragma unroll
    for (int i = 0; i < XR; ++i) xf[i] = bload128(rf, a.xscale ? x_src(i * nthr + tid) : kNoLoad, 0);
  }
  uint4 mv[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  {
    const brsrc_t rtab = make_rsrc(a.table, (uint32_t)a.Npad * (uint32_t)TB);
    const uint32_t o = tid < rw ? (uint32_t)(r0 + tid) * (uint32_t)TB : kNoLoad;
    if constexpr (TB == 2) {
      mv[0].x = bload16(rtab, o, 0);
    } else {
      mv[0] = bload128(rtab, o, 0);
      if constexpr (TB == 32) mv[1] = bload128(rtab, tid < rw ? o + 16u : kNoLoad, 0);
    }
  }

  // ---- LDS before the walk: activations (bf16: as fp16 with the row scale), LUT values / scales ----
  if constexpr (EDIT) {
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      if (a.clamp) xs[i] = clamp_act8<BF16>(xs[i], a.cval);
      if (a.xscale) xs[i] = scale_act8<BF16>(xs[i], xf[i]);
    }
  }
  float xunscale = 1.f;
  bool xfinite = true;
  if constexpr (BF16) {
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < XR; ++i) mx = xh_absmax2(mx, xs[i]);
    mx = wave_max_u32(max(mx & 0xFFFFu, mx >> 16) >> 1);
    uint32_t* smax = reinterpret_cast<uint32_t*>(sb + sa.lds_max);
    if (lane == 0) smax[wave] = mx;
    __syncthreads();
    uint32_t M16 = 0;
    for (int w = 0; w < wpg; ++w) M16 = max(M16, smax[w]);
    xfinite = M16 < 0x7F80u;
    const uint32_t emax = M16 >> 7, b = emax > 29u ? emax - 29u : 0u;
    xunscale = __uint_as_float((b + 15u) << 23);
#pragma unroll
    for (int i = 0; i < XR; ++i) xs[i] = xh_convert(xs[i], (b << 7) * 0x00010001u);
  }
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int s = i * nthr + tid;
    if (s < SM) *reinterpret_cast<uint4*>(sb + sa.lds_x + s * 16) = xs[i];
  }
  if (tid < rw) {
    if constexpr (TB == 2) {
      *reinterpret_cast<uint16_t*>(sb + sa.lds_meta + 2 * tid) = (uint16_t)mv[0].x;
    } else {
      *reinterpret_cast<uint4*>(sb + sa.lds_meta + TB * tid) = mv[0];
      if constexpr (TB == 32) *reinterpret_cast<uint4*>(sb + sa.lds_meta + TB * tid + 16) = mv[1];
    }
  }
  if constexpr (KIND == K_INT4_24) {
    if (tid < 16) stab[tid] = xsel_2_4_entry((uint32_t)tid);
  }
  __syncthreads();
  // LUT row tables from the staged values (LUT3: 64 pair entries; LUT4: 256)
  if constexpr (KIND == K_LUT3) {
    for (int i = tid; i < rw * 64; i += nthr) {
      const int q = i >> 6, e = i & 63;
      const uint16_t* lt = reinterpret_cast<const uint16_t*>(sb + sa.lds_meta + 16 * q);
      stab[i] = (uint32_t)lt[e & 7] | ((uint32_t)lt[e >> 3] << 16);
    }
  } else if constexpr (KIND == K_LUT4) {
    for (int i = tid; i < rw * 256; i += nthr) {
      const int q = i >> 8, e = i & 255;
      const uint16_t* lt = reinterpret_cast<const uint16_t*>(sb + sa.lds_meta + 32 * q);
      stab[i] = (uint32_t)lt[e & 15] | ((uint32_t)lt[e >> 4] << 16);
    }
  }
  if constexpr (LUT) __syncthreads();

  // ---- the loads of the walk, issued once the activations are staged (a
  // CU holds a bounded number of requests in flight: issued earlier, behind
  // the whole launch's code stream, they would hold up the staging) ----
  asm volatile("" ::: "memory");
  const brsrc_t rrp = make_rsrc(a.rowptr, has_csr ? (uint32_t)(a.N + 1) * 4u : 0u);
  const uint32_t rpv = bload32(rrp, tid <= rw ? (uint32_t)(r0 + tid) * 4u : kNoLoad, 0);
  uint4 kv[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  uint4 ksv = make_uint4(0, 0, 0, 0);
  const bool lr4 = a.lr_kind == CL_LR_INT4;
  if constexpr (LR) {
    const uint32_t rrb = (uint32_t)sa.rank_row_bytes, kb = (uint32_t)rw * rrb;
    const brsrc_t rR = make_rsrc(a.R, (uint32_t)a.Npad * rrb);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t o = 16u * (uint32_t)(tid + i * nthr);
      kv[i] = bload128(rR, o < kb ? (uint32_t)r0 * rrb + o : kNoLoad, 0);
    }
    const uint32_t sbytes = (uint32_t)rw * (uint32_t)sa.rsc_row_bytes;
    const brsrc_t rRs = make_rsrc(a.Rscale, lr4 ? (uint32_t)a.Npad * (uint32_t)sa.rsc_row_bytes : 0u);
    ksv = bload128(rRs, lr4 && (uint32_t)(16 * tid) < sbytes ? (uint32_t)r0 * (uint32_t)sa.rsc_row_bytes + 16u * (uint32_t)tid
                                                              : kNoLoad, 0);
  }
  const int nblk = (np + NB - 1) / NB;
  const brsrc_t rd = make_rsrc(a.dense, (uint32_t)a.Npad * (uint32_t)C * 16u);
  const brsrc_t rm = make_rsrc(a.meta, KIND == K_INT4_24 ? (uint32_t)a.Npad * (uint32_t)C * 8u : 0u);
  const uint32_t gchunk = (uint32_t)r0 * (uint32_t)C + (uint32_t)f0 + (uint32_t)lane;  // this lane's first chunk
  auto load_blk = [&](uint4 (&w)[NB], uint2 (&mw)[NB], int j) {
    // a pass past the slice loads nothing; lanes past the slice's end inside
    // its last pass read chunks of the next slice (or zero past the buffer) and are masked
    const uint32_t c0 = gchunk + (uint32_t)(j * NB * 64);
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const bool live = j * NB + q < np;
      w[q] = bload128_nt(rd, live ? (c0 + 64u * q) * 16u : kNoLoad, 0);
      if constexpr (KIND == K_INT4_24)
        mw[q] = bload64_nt(rm, live ? (c0 + 64u * q) * 8u : kNoLoad, 0);
      else
        mw[q] = make_uint2(0, 0);
    }
  };
  constexpr int NBUF = kStNBUF;
  uint4 W[NBUF][NB];
  uint2 MW[NBUF][NB];
#pragma unroll
  for (int b = 0; b < NBUF; ++b) load_blk(W[b], MW[b], b);
  // the workgroup's outliers (entries past out_cap are read from memory in
  // the finalisation).  Every load of the kernel is issued on every path (an
  // unused one reads nothing): the compiler's count of loads in flight then
  // stays exact, and no wait asks for more than the data it needs.
  uint32_t oc[kStOutLoads], ov[kStOutLoads];
  {
    const brsrc_t rcol = make_rsrc(a.col, has_csr ? (uint32_t)a.nnz * 4u : 0u);
    const brsrc_t rval = make_rsrc(a.val, has_csr ? (uint32_t)a.nnz * 2u : 0u);
#pragma unroll
    for (int i = 0; i < kStOutLoads; ++i) {
      const int j = tid + nthr * i, e = E0 + j;
      const bool ok = has_csr && e < E1 && j < sa.out_cap;
      oc[i] = bload32(rcol, ok ? (uint32_t)e * 4u : kNoLoad, 0);
      ov[i] = bload16(rval, ok ? (uint32_t)e * 2u : kNoLoad, 0);
    }
  }

  // ---- the walk: one chunk per lane per pass ----
  // The next row boundary B (a flat chunk index of the workgroup) and the row
  // n that ends there are wave-uniform; a lane's chunk f = f0 + 64 p + lane is
  // chunk f - (B - C) of row n when f < B, chunk f - B of row n + 1 otherwise.
  int n = f0 / C, B = (n + 1) * C;
  const int lxs = lane * XS;
  float acc = 0.f;
  auto deposit = [&](int row, float v) {  // this slice's partial sums of `row`
    const int off = row * C >= f0 ? sa.lds_part0 + row * 256 : sa.lds_part1 + wave * 256;
    *reinterpret_cast<float*>(sb + off + 4 * lane) = v;
  };
  auto pass = [&](const uint4& w, const uint2& mw, int p) {
    const int Pp = f0 + 64 * p;
    const int sB = B - Pp, sE = f1 - Pp;  // first lane of row n + 1 / past the slice
    const bool slow = sB < 64 || sE < 64;  // wave-uniform
    int xo = lxs + (Pp + C - B) * XS + sa.lds_x;
    uint32_t rb = (uint32_t)n * RTB;
    const bool nl = lane >= sB && lane < sE;  // in row n + 1
    if (slow) {
      if (nl) {
        xo -= C * XS;
        rb += RTB;
      }
      if (lane >= sE) xo = sa.lds_x;  // past the slice: any staged activation (the sum is masked)
    }
    uint32_t xv[P];
#pragma unroll
    for (int d = 0; d < XD; ++d) {
      const uint4 v = lds_u128(sdyn, (uint32_t)(xo + 16 * d));
      xv[4 * d] = v.x;
      xv[4 * d + 1] = v.y;
      xv[4 * d + 2] = v.z;
      xv[4 * d + 3] = v.w;
    }
    float t = slow ? 0.f : acc;
    if constexpr (KIND == K_INT4_24) {
      uint32_t qv[16], xg[16];
      int4_24_gather(stab, w, mw, xv, qv, xg);
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) t = mac2r<false>(qv[jj], xg[jj], t);
    } else {
      uint32_t wp[P];
      chunk_pairs<KIND, true>(stab, w, make_uint4(mw.x, mw.y, 0, 0), rb, 0u, wp);
#pragma unroll
      for (int jj = 0; jj < P; ++jj) t = mac2r<false>(wp[jj], xv[jj], t);
    }
    if (!slow) {
      acc = t;
    } else {
      if (lane >= sE) t = 0.f;
      if (sB < sE) {  // row n ends inside this pass
        deposit(n, nl ? acc : acc + t);
        acc = nl ? t : 0.f;
        ++n;
        B += C;
      } else {
        acc += t;
      }
    }
  };
  // A block with no row boundary and no slice end in it (the usual case) runs
  // as one straight stretch of code, so that the compiler can overlap one
  // pass's table lookups with the previous pass's multiply-adds.
  auto fast_pass = [&](const uint4& w, const uint2& mw, int p) {
    const int Pp = f0 + 64 * p;
    const uint32_t xo = (uint32_t)(lxs + (Pp + C - B) * XS + sa.lds_x);
    uint32_t xv[P];
#pragma unroll
    for (int d = 0; d < XD; ++d) {
      const uint4 v = lds_u128(sdyn, xo + 16u * d);
      xv[4 * d] = v.x;
      xv[4 * d + 1] = v.y;
      xv[4 * d + 2] = v.z;
      xv[4 * d + 3] = v.w;
    }
    if constexpr (KIND == K_INT4_24) {
      uint32_t qv[16], xg[16];
      int4_24_gather(stab, w, mw, xv, qv, xg);
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) acc = mac2r<false>(qv[jj], xg[jj], acc);
    } else {
      uint32_t wp[P];
      chunk_pairs<KIND, true>(stab, w, make_uint4(mw.x, mw.y, 0, 0), (uint32_t)n * RTB, 0u, wp);
#pragma unroll
      for (int jj = 0; jj < P; ++jj) acc = mac2r<false>(wp[jj], xv[jj], acc);
    }
  };
  auto comp_blk = [&](const uint4 (&w)[NB], const uint2 (&mw)[NB], int j) {
    const int P0 = f0 + 64 * NB * j;  // the block's first chunk
    if (B - P0 >= 64 * NB && f1 - P0 >= 64 * NB) {
#pragma unroll
      for (int q = 0; q < NB; ++q) fast_pass(w[q], mw[q], j * NB + q);
    } else {
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if (j * NB + q < np) pass(w[q], mw[q], j * NB + q);
    }
  };
  // Row pointers and rank-factor rows go to LDS now: they were asked for
  // before the code stream, so waiting for them waits for none of it (loads
  // complete in order), and their registers are free for the walk.  (They
  // are stored as loaded: an operation on them here would let the compiler
  // move it, and its wait, up to the loads.)
  if (tid <= rw) *reinterpret_cast<uint32_t*>(sb + sa.lds_rp + 4 * tid) = rpv;
  if constexpr (LR) {
    const uint32_t rrb = (uint32_t)sa.rank_row_bytes, kb = (uint32_t)rw * rrb;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t o = 16u * (uint32_t)(tid + i * nthr);
      // padded rows have a power-of-two length: row and offset by shifts
      const uint32_t lo = sa.rank_row_stride != sa.rank_row_bytes
                              ? (o >> __builtin_ctz(rrb)) * (uint32_t)sa.rank_row_stride + (o & (rrb - 1u))
                              : o;
      if (o < kb) *reinterpret_cast<uint4*>(sb + sa.lds_rank + lo) = kv[i];
    }
    if (lr4 && (uint32_t)(16 * tid) < (uint32_t)rw * (uint32_t)sa.rsc_row_bytes)
      *reinterpret_cast<uint4*>(sb + sa.lds_rsc + 16 * tid) = ksv;
  }
  // first round of blocks; then the outliers (asked for after the first
  // blocks of the code stream) go to LDS
#pragma unroll
  for (int b = 0; b < NBUF; ++b) {
    comp_blk(W[b], MW[b], b);
    load_blk(W[b], MW[b], b + NBUF);
  }
  if (has_csr) {
    uint16_t* ocol = reinterpret_cast<uint16_t*>(sb + sa.lds_out);
    uint16_t* oval = ocol + sa.out_cap;
#pragma unroll
    for (int i = 0; i < kStOutLoads; ++i) {
      const int j = tid + nthr * i;
      if (j < sa.out_cap) {
        ocol[j] = (uint16_t)oc[i];
        oval[j] = (uint16_t)ov[i];
      }
    }
  }
  for (int j0 = NBUF; j0 < nblk; j0 += NBUF) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      comp_blk(W[b], MW[b], j0 + b);
      load_blk(W[b], MW[b], j0 + b + NBUF);
    }
  }
  if (np > 0) deposit(n, acc);  // the slice's last row

  // ---- t = x' L_hat: the first wavefront adds up the prologue's tagged
  // partial sums (or reads t written by an earlier kernel) into LDS ----
  float* st = reinterpret_cast<float*>(sb + sa.lds_t);
  if constexpr (LR) {
    if (wave == 0) {
      const uint32_t target = a.lr_flag != nullptr ? lr_target(a.lr_flag, a.lr_epoch) : 0u;
      float tv[4];
      if (a.lr_flag != nullptr) {
        read_t_tagged(a.lrp.part, a.lrp.S, a.rank, lr_tag(a.lr_epoch, target), lane, a.lr_max_polls, a.lr_err, tv);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) tv[i] = lane + 64 * i < a.rank ? load_dev(a.t + lane + 64 * i) : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        if (j < a.rank) st[j] = tv[i];
      }
      if (a.lr_flag != nullptr && a.lr_epoch == 0) {  // recorded launch: this workgroup's reads of t are done
        __builtin_amdgcn_s_waitcnt(0);
        if (lane == 0) lr_reader_done(a.lr_flag, target, sa.lr_readers, wg);
      }
    }
  }
  __syncthreads();

  // ---- per row (eight threads each): partial sums, outliers, rank term ----
  auto x_lds = [&](int k) -> float {
    const int c = k / SPAN, o = k - c * SPAN;
    return act_f32<false>(lds_u16(sdyn, (uint32_t)(sa.lds_x + c * XS + 2 * o)));  // fp16 (bf16 rows were converted)
  };
  // Outlier entry e of the workgroup (e < out_cap: staged in LDS), its value
  // times its activation added to v.  The staged and the unstaged entries
  // are read in loops of their own: one expression for both would read
  // through a generic pointer (a flat load, waited for with every other
  // memory access, for every entry).
  auto outlier_lds = [&](int e, float v) -> float {
    const uint32_t c = lds_u16(sdyn, (uint32_t)(sa.lds_out + 2 * e));
    const uint32_t vb = lds_u16(sdyn, (uint32_t)(sa.lds_out + 2 * sa.out_cap + 2 * e));
    return __builtin_fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)vb), x_lds((int)c), v);
  };
  auto outlier_mem = [&](int e, float v) -> float {
    return __builtin_fmaf((float)__builtin_bit_cast(_Float16, a.val[E0 + e]), x_lds((int)a.col[E0 + e]), v);
  };
  auto rank_term = [&](int rl, int j, float v) -> float {  // v + R^T[row rl][j] (staged in LDS) * t_j
    const uint8_t* rrow = sb + sa.lds_rank + rl * sa.rank_row_stride;
    float rvv;
    if (lr4) {
      const uint32_t byte = rrow[j >> 1];
      const uint32_t jg = ((uint32_t)j * a.group_mul) >> 16;
      const uint16_t sc = *reinterpret_cast<const uint16_t*>(sb + sa.lds_rsc + rl * sa.rsc_row_bytes + 2 * jg);
      rvv = (float)((int)((byte >> (4 * (j & 1))) & 0xFu) - 8) * (float)__builtin_bit_cast(_Float16, sc);
    } else {
      const uint32_t uu = *reinterpret_cast<const uint16_t*>(rrow + 2 * j);
      rvv = a.lr_kind == CL_LR_BF16 ? __uint_as_float(uu << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)uu);
    }
    return __builtin_fmaf(st[j], rvv, v);
  };
  // Rows of more than 64 outliers on average: a wavefront per row (the
  // workgroup's wavefronts take its rows in turn), a lane per outlier and per
  // rank term.  (Measured on 28672 -> 8192 with 129 outliers a row: about 1 us
  // faster than eight threads per row; rows of 37 outliers are not.)
  if (E1 - E0 > 64 * rw) {
    for (int rl = wave; rl < rw; rl += wpg) {
      float v = *reinterpret_cast<const float*>(sb + sa.lds_part0 + rl * 256 + 4 * lane);
      const int w1 = rl * C / Lw + 1;
      if (w1 * Lw < (rl + 1) * C) v += *reinterpret_cast<const float*>(sb + sa.lds_part1 + w1 * 256 + 4 * lane);
      if constexpr (!LUT)
        v *= (float)__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(sb + sa.lds_meta + 2 * rl));
      if (has_csr) {
        const int e0 = (int)*reinterpret_cast<const uint32_t*>(sb + sa.lds_rp + 4 * rl) - E0;
        const int e1 = (int)*reinterpret_cast<const uint32_t*>(sb + sa.lds_rp + 4 * rl + 4) - E0;
        const int es = min(e1, sa.out_cap);
        int e = e0 + lane;
        for (; e < es; e += 64) v = outlier_lds(e, v);
        for (; e < e1; e += 64) v = outlier_mem(e, v);
      }
      if constexpr (BF16) v = xfinite ? v * xunscale : __builtin_nanf("");
      if constexpr (LR)
        for (int j = lane; j < a.rank; j += 64) v = rank_term(rl, j, v);
      // the row's sum: quad swaps, mirrored quads, mirrored halves of each
      // 16-lane row, then across the rows
      v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
      v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
      v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
      v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (lane == 0) a.y[r0 + rl] = v;
    }
    return;
  }
  const int u = tid & 7;
  for (int rb0 = 0; rb0 < rw; rb0 += nthr >> 3) {
    const int rl = rb0 + (tid >> 3);
    float v = 0.f;
    if (rl < rw) {
      const float4 pa = *reinterpret_cast<const float4*>(sb + sa.lds_part0 + rl * 256 + 32 * u);
      const float4 pb = *reinterpret_cast<const float4*>(sb + sa.lds_part0 + rl * 256 + 32 * u + 16);
      v = ((pa.x + pa.y) + (pa.z + pa.w)) + ((pb.x + pb.y) + (pb.z + pb.w));
      const int w1 = rl * C / Lw + 1;  // the slice that may start inside the row
      if (w1 * Lw < (rl + 1) * C) {
        const float4 qa = *reinterpret_cast<const float4*>(sb + sa.lds_part1 + w1 * 256 + 32 * u);
        const float4 qb = *reinterpret_cast<const float4*>(sb + sa.lds_part1 + w1 * 256 + 32 * u + 16);
        v += ((qa.x + qa.y) + (qa.z + qa.w)) + ((qb.x + qb.y) + (qb.z + qb.w));
      }
      if constexpr (!LUT)
        v *= (float)__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(sb + sa.lds_meta + 2 * rl));
      if (has_csr) {
        const int e0 = (int)*reinterpret_cast<const uint32_t*>(sb + sa.lds_rp + 4 * rl) - E0;
        const int e1 = (int)*reinterpret_cast<const uint32_t*>(sb + sa.lds_rp + 4 * rl + 4) - E0;
        const int es = min(e1, sa.out_cap);
        int e = e0 + u;
        for (; e < es; e += 8) v = outlier_lds(e, v);
        for (; e < e1; e += 8) v = outlier_mem(e, v);
      }
      if constexpr (BF16) v = xfinite ? v * xunscale : __builtin_nanf("");
      if constexpr (LR) {
        const int rpt = a.rank >> 3;  // rank terms a thread: a contiguous run of them
        const uint32_t rrow = (uint32_t)(sa.lds_rank + rl * sa.rank_row_stride);
        if (!lr4 && (a.rank & 31) == 0) {  // 16-bit factors, four terms at a time
          for (int j = u * rpt; j < (u + 1) * rpt; j += 4) {
            const uint2 r4 = lds_u64(sdyn, rrow + 2 * j);
            const float4 t4 = *reinterpret_cast<const float4*>(st + j);
            const uint32_t rr[2] = {r4.x, r4.y};
            float f[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t h = (rr[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
              f[q] = a.lr_kind == CL_LR_BF16 ? __uint_as_float(h << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
            }
            v = __builtin_fmaf(t4.x, f[0], v);
            v = __builtin_fmaf(t4.y, f[1], v);
            v = __builtin_fmaf(t4.z, f[2], v);
            v = __builtin_fmaf(t4.w, f[3], v);
          }
        } else if (lr4 && (a.rank & 63) == 0 && (a.group & 7) == 0) {  // int4 factors, eight terms (one scale) at a time
          for (int j = u * rpt; j < (u + 1) * rpt; j += 8) {
            const uint32_t b8 = lds_u32(sdyn, rrow + j / 2);
            const uint32_t jg = ((uint32_t)j * a.group_mul) >> 16;
            const float sc = (float)__builtin_bit_cast(
                _Float16, (uint16_t)lds_u16(sdyn, (uint32_t)(sa.lds_rsc + rl * sa.rsc_row_bytes + 2 * jg)));
            const float4 t0 = *reinterpret_cast<const float4*>(st + j), t1 = *reinterpret_cast<const float4*>(st + j + 4);
            const float tq[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
            for (int q = 0; q < 8; ++q) v = __builtin_fmaf(tq[q], (float)((int)((b8 >> (4 * q)) & 0xFu) - 8) * sc, v);
          }
        } else {
          for (int j = u; j < a.rank; j += 8) v = rank_term(rl, j, v);
        }
      }
    }
    // the eight threads of the row: quad swaps, then the mirrored quad of each half row
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
    if (u == 0 && rl < rw) a.y[r0 + rl] = v;
  }
}

template <int KIND, bool BF16, int XR, bool LR>
static void launch_stream_e(const StreamArgs& s, int grid, int threads, int lds, hipStream_t st) {
  if (s.r.clamp || s.r.xscale)
    hipLaunchKernelGGL((decode_stream_kernel<KIND, BF16, XR, LR, true>), dim3(grid), dim3(threads), lds, st, s);
  else
    hipLaunchKernelGGL((decode_stream_kernel<KIND, BF16, XR, LR, false>), dim3(grid), dim3(threads), lds, st, s);
}

template <int KIND, bool BF16, int XR>
static void launch_stream_l(const StreamArgs& s, int grid, int threads, int lds, hipStream_t st) {
  if (s.r.lr_kind != CL_LR_NONE) launch_stream_e<KIND, BF16, XR, true>(s, grid, threads, lds, st);
  else launch_stream_e<KIND, BF16, XR, false>(s, grid, threads, lds, st);
}

// Staging slots per thread of one activation row (the host rejects plans above 12).
template <int KIND>
inline int stream_slots_per_thread(int chunks, int threads) {
  return (chunks * RowX<KIND>::slots + threads - 1) / threads;
}

template <int KIND, bool BF16>
static hipError_t launch_stream_t(const StreamArgs& s, int grid, int threads, int lds, hipStream_t st) {
  const int per = stream_slots_per_thread<KIND>(s.r.chunks, threads);
  if (per <= 2) launch_stream_l<KIND, BF16, 2>(s, grid, threads, lds, st);
  else if (per <= 4) launch_stream_l<KIND, BF16, 4>(s, grid, threads, lds, st);
  else if (per <= 8) launch_stream_l<KIND, BF16, 8>(s, grid, threads, lds, st);
  else if (per <= 12) launch_stream_l<KIND, BF16, 12>(s, grid, threads, lds, st);
  else return hipErrorInvalidConfiguration;
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_stream_kind(const StreamArgs& s, int grid, int threads, int lds, bool bf16, hipStream_t st) {
  return bf16 ? launch_stream_t<KIND, true>(s, grid, threads, lds, st) : launch_stream_t<KIND, false>(s, grid, threads, lds, st);
}

}  // namespace cl
