// decode_rows.h -- batch 1..4 forward: a wavefront per group of rows, lanes along K.
//
// The bandwidth-bound decode path.  A workgroup of four wavefronts owns 4*R
// consecutive rows; wavefront w owns R of them and streams their whole K range:
// in pass p, lane l takes chunk 64p + l of each of its R rows (the row-major
// layout makes that one contiguous 1 KiB load per row), dequantises it through
// the row's LUT table in LDS, and multiplies with the activations of that chunk.
// The 64 lane partials of a row are summed with cross-lane shuffles at the end:
// no cross-workgroup reduction.
//
// Each wavefront moves only a few KiB, so the kernel is shaped around latency:
// every load a wavefront needs is issued before it waits for any of them --
// LUT values, the activation staging, the first two blocks of NB passes of
// the code stream, the outlier heads and rank factors -- as a fixed sequence of
// buffer loads without branches (an element that does not exist gets an
// offset past the buffer, which reads zero).  The compiler can then count the
// loads exactly and wait for each block just before it is used, so the
// dequantisation of the first rows overlaps the arrival of the rest.
//
// The activations are staged once per workgroup in LDS (chunk c of row m at
// c * XS bytes, XS the chunk's activation bytes padded so that eight lanes'
// 16-byte reads fall in distinct banks), which keeps them out of the registers
// and lets the outlier gather read LDS instead of memory.  At batch 1 the
// kernel also takes raw activations of a layer that clamps them ("Compressing
// Large Language Models by Joint Sparsification and Quantization", Approach)
// or scales some channels ("SLiM" page, rebuttal section "Output Error
// Minimization in SLiM-Quant") and edits them on their way to LDS, which saves
// a prep kernel's launch.  The row tables are
// the kernel's only static LDS array, at address 0, so the table addresses
// built from the packed bytes are absolute.
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
#include "lowrank.h"
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
  uint32_t group_mul;  // ceil(2^16 / group): (j * group_mul) >> 16 == j / group for every rank index j < 256
  int Npad;   // rows with storage (a multiple of 64)
  int nnz;    // outliers in the layer
  int npass;  // ceil(chunks / 64)
  int xrow;   // LDS bytes per staged activation row (npass * 64 chunks)
  int lds_x;  // byte offset of the staged activations in the dynamic LDS
  // Low-rank prologue in the same launch: workgroups [0, lr_wgs) compute t
  // (lr_mode 0 or 1, blocks S x lr_ntj x activation tiles) and publish
  // lr_epoch, or for lr_epoch 0 (a launch recorded into a graph) the launch's
  // generation (lr_target); the row workgroups wait for it before reading t
  // and, in a recorded launch, count themselves done afterwards.
  // lr_wgs = 0: t was computed by an earlier kernel (lr_flag NULL).
  LrSplitArgs lrp;
  int lr_wgs, lr_ntj, lr_mode;
  uint32_t* lr_flag;
  uint32_t lr_epoch;
  uint32_t lr_max_polls;  // bound of the wait for t
  uint32_t* lr_err;       // set when a wait gives up (host memory)
  // raw activations (ldx = K): clamp them to [-cval, cval] and multiply them by
  // the per-channel factors xscale ([K] fp16; NULL: none) while staging them
  int clamp;
  float cval;
  const uint16_t* xscale;
};

// LDS bytes per chunk of staged activations: the chunk's 2 * span bytes padded
// so that the stride in dwords is 4 * (odd number) and lanes 0..7 of a 128-bit
// read hit 8 distinct groups of four banks.
template <int KIND>
struct RowX {
  static constexpr int span = KindTraits<KIND>::span;
  static constexpr int stride = span == 40 ? 80 : span == 32 ? 80 : span == 64 ? 144 : 48;
  static constexpr int slots = stride / 16;  // 16-byte slots per chunk
};

// Static LDS of the row tables: per wavefront R row tables (LUT3: 64 pair
// entries, 256 bytes; LUT4: 256 pair entries, 1 KiB), the shared 2:4 selector
// table, or a token array.
template <int KIND, int R>
constexpr int row_tab_bytes() {
  return (KIND == K_LUT3 || KIND == K_LUT4) ? 4 * R * row_table_bytes<KIND>() : KIND == K_INT4_24 ? 256 : 16;
}

// 16-byte activation slots each thread stages per round (the first round is
// issued before the code stream, further rounds after it).
template <int MB>
constexpr int row_x_rounds() { return MB <= 2 ? 8 : 12; }
// Slots per thread that one staging round of one activation row may hold: the
// round that edits raw activations, or converts bf16 ones (all of the row).
template <bool BF16>
constexpr int row_x_slots1() { return BF16 ? 16 : 8; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <bool BF16>
__device__ __forceinline__ float act_f32(uint32_t v16) {
  if constexpr (BF16) return __uint_as_float(v16 << 16);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)v16);
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

// bf16 activations of a batch-1 row staged as fp16 (the multiply-adds then run
// as fp16 dot products, one instruction per weight pair, instead of two mixed
// fp16 x bf16 multiply-adds and conversions): every value is multiplied by the
// same power of two 2^(112 - b), chosen from the row's largest exponent e_max
// so that the largest magnitude lands in [2^14, 2^15) (b = max(e_max - 29, 0)),
// and the row's sum is multiplied back by 2^(b - 112) before the rank term.
// A bf16 value (8 significant bits) whose scaled exponent stays in fp16's
// normal range is exact; so is a bf16 subnormal when b = 0.  Values more than
// 2^29 below the row's largest are replaced by a value within 2^-14 of them in
// scaled units (less than 2^-28 of the row's largest magnitude).
typedef unsigned short xh_u16x2 __attribute__((ext_vector_type(2)));
// packed 16-bit maxima of 2|bf16| (the bits shifted left by one drop the sign;
// a form of its own, so that the compiler does not keep the conversion's
// masked values alive from here to the conversion)
__device__ __forceinline__ uint32_t xh_absmax2(uint32_t m, uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const xh_u16x2 one = {1, 1};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    m = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(xh_u16x2, m),
                                                               (xh_u16x2)(__builtin_bit_cast(xh_u16x2, w[i]) << one)));
  return m;
}
// maximum over the wavefront: rotations inside rows of 16 lanes, then the four rows
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x124, 0xF, 0xF, false));  // row_ror 4
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x128, 0xF, 0xF, false));  // row_ror 8
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)m, 32), (uint32_t)__builtin_amdgcn_readlane((int)m, 48)));
}
// |bf16| bits minus b << 7 in each half (saturating at 0) is the fp16 exponent
// and the top 7 significand bits, three places to the right; the sign is kept.
__device__ __forceinline__ uint4 xh_convert(uint4 v, uint32_t sub2) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const xh_u16x2 d = __builtin_elementwise_sub_sat(__builtin_bit_cast(xh_u16x2, w[i] & 0x7FFF7FFFu),
                                                     __builtin_bit_cast(xh_u16x2, sub2));
    const xh_u16x2 three = {3, 3};
    w[i] = (w[i] & 0x80008000u) | __builtin_bit_cast(uint32_t, (xh_u16x2)(d << three));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint4 lds_u128(const uint32_t* lds, uint32_t byte_addr) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(lds) + byte_addr);
}

// R = rows per wavefront, MB = activation rows (M <= MB), NB = passes per block,
// XR = activation slots staged per thread, LR = the layer has a low-rank part
// (a template parameter so that layers without one carry no conditional loads,
// which would make the compiler's load counting conservative).
template <int KIND, int MB, bool BF16, int R, int NB, int XR, bool LR, bool EDIT>
__global__ void __launch_bounds__(256) decode_rows_kernel(RowArgs a) {
  constexpr int SPAN = KindTraits<KIND>::span, P = KindTraits<KIND>::pairs, XD = SPAN / 8;  // 16-byte x slots per chunk
  constexpr int XS = RowX<KIND>::stride, XSL = RowX<KIND>::slots;
  constexpr bool LUT = KIND == K_LUT3 || KIND == K_LUT4;
  // bf16 activations of one row: staged as fp16 with a row scale (one staging
  // round holds the whole row; the host checks it)
  constexpr bool XH = BF16 && MB == 1;
  constexpr bool XB = BF16 && !XH;  // bf16 values in LDS (multiply-adds in fp32)
  constexpr uint32_t RTB = (uint32_t)row_table_bytes<KIND>();  // bytes of one row table
  constexpr int XMAXW = row_tab_bytes<KIND, R>() / 4;          // after the tables: the waves' row maxima
  __shared__ __attribute__((aligned(16))) uint32_t stab[row_tab_bytes<KIND, R>() / 4 + 4];  // at LDS address 0
  extern __shared__ __attribute__((aligned(16))) uint32_t sdyn[];                      // t, then the activations
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  if constexpr (LR) {
    if ((int)blockIdx.x < a.lr_wgs) {  // a prologue workgroup; MB is its activation tile
      const int b = blockIdx.x, S = a.lrp.S, s = b % S, tj = (b / S) % a.lr_ntj, tm = b / (S * a.lr_ntj);
      uint8_t* smem = reinterpret_cast<uint8_t*>(sdyn);
      if (a.lr_mode == 0) lr_split_block<0, MB, BF16, EDIT>(a.lrp, s, tj, tm, a.lr_ntj, smem);
      else lr_split_block<1, MB, BF16, EDIT>(a.lrp, s, tj, tm, a.lr_ntj, smem);
      return;
    }
  }
  const int rb = (int)blockIdx.x - (LR ? a.lr_wgs : 0);
  const int row0 = (rb * 4 + wave) * R;  // rows row0 + r >= Npad read zeros and are not stored
  const uint32_t tabbase = (uint32_t)wave * R * RTB;
  const bool has_csr = a.rowptr != nullptr;
  constexpr bool has_lr = LR;

  // ---- row pointers: vector loads of uniform addresses, issued first so that
  // the outlier heads wait for them alone (scalar loads would hold back every
  // load behind one all-or-nothing wait); no outliers: zeros ----
  int e0[R], e1[R];
  {
    const brsrc_t rrp = make_rsrc(a.rowptr, has_csr ? (uint32_t)(a.N + 1) * 4u : 0u);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      e0[r] = (int)bload32(rrp, (uint32_t)min(row0 + r, a.N) * 4u, 0);
      e1[r] = (int)bload32(rrp, (uint32_t)min(row0 + r + 1, a.N) * 4u, 0);
    }
  }

  // ---- LUT values or integer row scales ----
  // LUT4: lane l builds pair entries 4l..4l+3 = lut[4 (l & 3) + j] | lut[l >> 2] << 16.
  // LUT3: lane l builds pair entry l = lut[l & 7] | lut[l >> 3] << 16.
  constexpr uint32_t TB = KIND == K_LUT4 ? 32u : KIND == K_LUT3 ? 16u : 2u;  // table bytes per row
  const brsrc_t rtab = make_rsrc(a.table, (uint32_t)a.Npad * TB);
  uint32_t tva[R], tvb[R];
  uint2 tv4[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t rb = (uint32_t)(row0 + r) * TB;
    if constexpr (KIND == K_LUT4) {
      tv4[r] = bload64(rtab, rb + 8u * (lane & 3), 0);
      tva[r] = bload16(rtab, rb + 2u * (lane >> 2), 0);
      tvb[r] = 0;
    } else if constexpr (KIND == K_LUT3) {
      tva[r] = bload16(rtab, rb + 2u * (lane & 7), 0);
      tvb[r] = bload16(rtab, rb + 2u * (lane >> 3), 0);
      tv4[r] = make_uint2(0, 0);
    } else {
      tva[r] = bload16(rtab, rb, 0);
      tvb[r] = 0;
      tv4[r] = make_uint2(0, 0);
    }
  }

  // ---- activations (and t): the workgroup stages them in LDS, zero past K and past M ----
  // Slot s of the staged activations is LDS byte lds_x + 16 s (rows of
  // npass * 64 chunks of XSL slots each, back to back); its activation row m
  // takes at most three compares and its chunk a division by a constant.
  const int SM = a.npass * 64 * XSL;  // slots per activation row
  const int xslots = MB * SM;
  const brsrc_t rx = make_rsrc(a.x, (uint32_t)a.M * (uint32_t)a.ldx * 2u);
  // byte offset of slot s in x (kNoLoad for a zero slot); fac: of its factors instead
  auto x_src = [&](int s, bool fac = false) -> uint32_t {
    int m = 0;
    if constexpr (MB > 1) m = (s >= SM) + (MB > 2 ? (s >= 2 * SM) + (s >= 3 * SM) : 0);
    const int rem = s - m * SM, c = rem / XSL, d = rem - c * XSL, k = c * SPAN + 8 * d;
    const bool ok = s < xslots && d < XD && m < a.M && k < a.ldx;  // ldx: a multiple of 8, zero past K
    return ok ? (fac ? (uint32_t)k * 2u : ((uint32_t)m * (uint32_t)a.ldx + (uint32_t)k) * 2u) : kNoLoad;
  };
  uint4 xs[XR];
#pragma unroll
  for (int i = 0; i < XR; ++i) xs[i] = bload128(rx, x_src(i * 256 + tid), 0);
  // EDIT: raw activations; their per-channel factors load beside them and both
  // are consumed where the activations go to LDS, after the code stream is
  // issued (measured faster than editing them before it, which exposes one
  // load latency, and than a prep kernel of its own)
  uint4 xf[EDIT ? XR : 1];
  if constexpr (EDIT) {
    const brsrc_t rf = make_rsrc(a.xscale, a.xscale ? (uint32_t)a.ldx * 2u : 0u);
#pragma unroll
    for (int i = 0; i < XR; ++i) xf[i] = a.xscale ? bload128(rf, x_src(i * 256 + tid, true), 0) : make_uint4(0, 0, 0, 0);
  }

  // ---- the code stream: blocks of NB passes, two in flight ----
  const int nblk = (a.npass + NB - 1) / NB;
  const brsrc_t rd = make_rsrc(a.dense, (uint32_t)a.Npad * (uint32_t)a.chunks * 16u);
  const brsrc_t rm = make_rsrc(a.meta, KIND == K_INT4_24 ? (uint32_t)a.Npad * (uint32_t)a.chunks * 8u : 0u);
  auto load_blk = [&](uint4 (&w)[NB][R], uint2 (&mw)[NB][R], int b) {
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int c = (b * NB + q) * 64 + lane;
      const bool okc = b < nblk && c < a.chunks;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t idx = (uint32_t)(row0 + r) * (uint32_t)a.chunks + (uint32_t)c;  // rows past Npad: out of range
        w[q][r] = bload128_nt(rd, okc ? idx * 16u : kNoLoad, 0);
        if constexpr (KIND == K_INT4_24)
          mw[q][r] = bload64_nt(rm, okc ? idx * 8u : kNoLoad, 0);
        else
          mw[q][r] = make_uint2(0, 0);
      }
    }
  };
  uint4 WA[NB][R], WB[NB][R];
  uint2 MA[NB][R], MB_[NB][R];
  load_blk(WA, MA, 0);
  load_blk(WB, MB_, 1);

  // ---- outlier heads and rank factors (consumed at the end) ----
  const brsrc_t rcol = make_rsrc(a.col, (uint32_t)a.nnz * 4u), rval = make_rsrc(a.val, (uint32_t)a.nnz * 2u);
  int ccol[R];
  float cval[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = e0[r] + lane;
    const bool ok = e < e1[r];
    ccol[r] = (int)bload32(rcol, ok ? (uint32_t)e * 4u : kNoLoad, 0);
    cval[r] = (float)__builtin_bit_cast(_Float16, (uint16_t)bload16(rval, ok ? (uint32_t)e * 2u : kNoLoad, 0));
  }
  float rv[R][4];
  if constexpr (LR) {
    const bool lr4 = a.lr_kind == CL_LR_INT4;
    const int gr = lr4 ? (a.rank + a.group - 1) / a.group : 1;
    const brsrc_t rR = make_rsrc(a.R, (uint32_t)a.Npad * (uint32_t)(lr4 ? (a.rank + 1) / 2 : a.rank * 2));
    const brsrc_t rRs = make_rsrc(a.Rscale, lr4 ? (uint32_t)a.Npad * (uint32_t)gr * 2u : 0u);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        const uint32_t n = (uint32_t)(row0 + r);
        const bool ok = j < a.rank;  // rows past Npad are out of range
        const uint32_t jg = ((uint32_t)j * a.group_mul) >> 16;  // j / group (int4 scales)
        // int4: R^T codes [Npad][ceil(r/2)], scales [Npad][ceil(r/g)]; else R^T [Npad][r] 16-bit
        const uint32_t byte = bload8(rR, ok && lr4 ? n * (uint32_t)((a.rank + 1) >> 1) + (uint32_t)(j >> 1) : kNoLoad, 0);
        const uint32_t sc = bload16(rRs, ok && lr4 ? (n * (uint32_t)gr + jg) * 2u : kNoLoad, 0);
        const uint32_t u = bload16(rR, ok && !lr4 ? (n * (uint32_t)a.rank + (uint32_t)j) * 2u : kNoLoad, 0);
        const int qv = (int)((byte >> (4 * (j & 1))) & 0xFu) - 8;
        const float v4 = ok ? (float)qv * (float)__builtin_bit_cast(_Float16, (uint16_t)sc) : 0.f;
        const float v16 = a.lr_kind == CL_LR_BF16 ? __uint_as_float(u << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)u);
        rv[r][i] = lr4 ? v4 : v16;
      }
  }

  // ---- LDS: activations, t, tables ----
  if constexpr (EDIT) {
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      if (a.clamp) xs[i] = clamp_act8<BF16>(xs[i], a.cval);
      if (a.xscale) xs[i] = scale_act8<BF16>(xs[i], xf[i]);
    }
  }
  float xunscale = 1.f;  // XH: 2^(b - 112), the inverse of the staging scale
  bool xfinite = true;
  if constexpr (XH) {
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < XR; ++i) mx = xh_absmax2(mx, xs[i]);  // slots past the row read zero
    mx = wave_max_u32(max(mx & 0xFFFFu, mx >> 16) >> 1);
    if (lane == 0) stab[XMAXW + wave] = mx;
    __syncthreads();
    const uint32_t M16 = max(max(stab[XMAXW], stab[XMAXW + 1]), max(stab[XMAXW + 2], stab[XMAXW + 3]));
    xfinite = M16 < 0x7F80u;  // an infinite or NaN activation makes every output of the row NaN
    const uint32_t emax = M16 >> 7, b = emax > 29u ? emax - 29u : 0u;
    xunscale = __uint_as_float((b + 15u) << 23);
#pragma unroll
    for (int i = 0; i < XR; ++i) xs[i] = xh_convert(xs[i], (b << 7) * 0x00010001u);
  }
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int s = i * 256 + tid;
    if (s < xslots) *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(sdyn) + a.lds_x + s * 16) = xs[i];
  }
  // activation blocks larger than one round of XR slots per thread: further
  // rounds, loaded after the code stream is in flight (their wait covers it);
  // never with edits (the host sends such blocks through the prep kernel),
  // never with bf16 activations at batch 1 (one round holds the row)
  for (int base = XR * 256; !XH && base < xslots; base += XR * 256) {
#pragma unroll
    for (int i = 0; i < XR; ++i) xs[i] = bload128(rx, x_src(base + i * 256 + tid), 0);
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int s = base + i * 256 + tid;
      if (s < xslots) *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(sdyn) + a.lds_x + s * 16) = xs[i];
    }
  }
  if constexpr (KIND == K_LUT4) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t hi = tva[r] << 16;
      *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(stab) + tabbase + r * RTB + 16 * lane) =
          make_uint4((tv4[r].x & 0xFFFFu) | hi, (tv4[r].x >> 16) | hi, (tv4[r].y & 0xFFFFu) | hi, (tv4[r].y >> 16) | hi);
    }
  } else if constexpr (KIND == K_LUT3) {
#pragma unroll
    for (int r = 0; r < R; ++r) stab[(tabbase >> 2) + r * 64 + lane] = tva[r] | (tvb[r] << 16);
  } else if constexpr (KIND == K_INT4_24) {
    if (tid < 16) {
      const uint2 e = seltab_2_4_entry((uint32_t)tid);
      stab[2 * tid] = e.x;
      stab[2 * tid + 1] = e.y;
    }
  }
  __syncthreads();

  // ---- dequantise and multiply ----
  float acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[r][m] = 0.f;
  auto comp_blk = [&](const uint4 (&w)[NB][R], const uint2 (&mw)[NB][R], int b) {
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int p = b * NB + q;
      if (p < a.npass) {
        const int c = p * 64 + lane;
        uint32_t xv[MB][P];
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int d = 0; d < XD; ++d) {
            const uint4 v = lds_u128(sdyn, (uint32_t)(a.lds_x + m * a.xrow + c * XS + 16 * d));
            xv[m][4 * d] = v.x;
            xv[m][4 * d + 1] = v.y;
            xv[m][4 * d + 2] = v.z;
            xv[m][4 * d + 3] = v.w;
          }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint32_t wp[P];
          chunk_pairs<KIND, true>(stab, w[q][r], make_uint4(mw[q][r].x, mw[q][r].y, 0, 0), tabbase + (uint32_t)r * RTB,
                                  0u, wp);
#pragma unroll
          for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int j = 0; j < P; ++j) acc[r][m] = mac2r<XB>(wp[j], xv[m][j], acc[r][m]);
        }
      }
    }
  };
  // the first two blocks outside the loop, so that their waits are exact
  comp_blk(WA, MA, 0);
  load_blk(WA, MA, 2);
  comp_blk(WB, MB_, 1);
  load_blk(WB, MB_, 3);
  for (int b = 2; b < nblk; b += 2) {
    comp_blk(WA, MA, b);
    load_blk(WA, MA, b + 2);
    comp_blk(WB, MB_, b + 1);
    load_blk(WB, MB_, b + 3);
  }

  // ---- integer formats: the row scale multiplies the dense part only ----
  if constexpr (!LUT) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)tva[r]);
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[r][m] *= sc;
    }
  }
  // ---- outliers: activations gathered from LDS ----
  auto x_lds = [&](int m, int k) -> float {
    const int c = k / SPAN, o = k - c * SPAN;
    return act_f32<XB>(lds_u16(sdyn, (uint32_t)(a.lds_x + m * a.xrow + c * XS + 2 * o)));
  };
  if (has_csr) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[r][m] = __builtin_fmaf(cval[r], x_lds(m, ccol[r]), acc[r][m]);
      for (int e = e0[r] + 64 + lane; e < e1[r]; e += 64) {
        const float v = (float)__builtin_bit_cast(_Float16, a.val[e]);
        const int cc = a.col[e];
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[r][m] = __builtin_fmaf(v, x_lds(m, cc), acc[r][m]);
      }
    }
  }
  if constexpr (XH) {  // back from the staging scale (exact: a power of two), before the rank term
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = xfinite ? acc[r][0] * xunscale : __builtin_nanf("");
  }
  // ---- rank terms: t (LDS) times R^T ----
  if constexpr (LR) {
    // t is ready once the prologue (earlier kernel, or this launch's first
    // workgroups) has published it; read through the coherent path
    const uint32_t target = a.lr_flag != nullptr ? lr_target(a.lr_flag, a.lr_epoch) : 0u;
    const bool t_ok =
        a.lr_flag == nullptr || wait_lowrank(lr_word(a.lr_flag, a.lr_epoch), target, lane, a.lr_max_polls, a.lr_err);
    float tv[MB][4];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        tv[m][i] = (j < a.rank && m < a.M) ? (t_ok ? load_dev(a.t + (size_t)m * a.rank + j) : __builtin_nanf("")) : 0.f;
      }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[r][m] = __builtin_fmaf(tv[m][i], rv[r][i], acc[r][m]);
    if (a.lr_flag != nullptr && a.lr_epoch == 0) {  // recorded launch: the workgroup's reads of t are done
      __syncthreads();
      if (tid == 0) lr_reader_done(a.lr_flag, target, (int)gridDim.x - a.lr_wgs, (int)blockIdx.x - a.lr_wgs);
    }
  }
  // ---- reduce over the lanes and store ----
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const float v = wave_sum(acc[r][m]);
      const int row = row0 + r;
      if (lane == 0 && m < a.M && row < a.N) a.y[(size_t)m * a.N + row] = v;
    }
}

// Largest dynamic LDS a row-wise workgroup may take; larger activation blocks go to the tile kernel.
constexpr int kRowsMaxLds = 64 * 1024;

template <int KIND, int MB>
inline int rows_lds_layout(RowArgs& a) {
  a.npass = (a.chunks + 63) / 64;
  a.xrow = a.npass * 64 * RowX<KIND>::stride;
  a.lds_x = 0;
  const int lds = MB * a.xrow;
  const int lr = a.lr_wgs > 0 ? lr_scratch_bytes(a.lr_mode, MB) : 0;  // prologue workgroups reuse it
  return lds > lr ? lds : lr;
}

// Passes per block: one when a row takes at most two passes (both blocks then
// hold real chunks), else two.
template <int KIND, int MB, bool BF16, int R, int XR, bool EDIT>
static void launch_rows_xe(const RowArgs& a, int grid, int lds, hipStream_t st) {
  const bool lr = a.lr_kind != CL_LR_NONE;
  if (a.npass <= 2) {
    if (lr) hipLaunchKernelGGL((decode_rows_kernel<KIND, MB, BF16, R, 1, XR, true, EDIT>), dim3(grid), dim3(256), lds, st, a);
    else hipLaunchKernelGGL((decode_rows_kernel<KIND, MB, BF16, R, 1, XR, false, EDIT>), dim3(grid), dim3(256), lds, st, a);
  } else {
    if (lr) hipLaunchKernelGGL((decode_rows_kernel<KIND, MB, BF16, R, 2, XR, true, EDIT>), dim3(grid), dim3(256), lds, st, a);
    else hipLaunchKernelGGL((decode_rows_kernel<KIND, MB, BF16, R, 2, XR, false, EDIT>), dim3(grid), dim3(256), lds, st, a);
  }
}

// Kernels that edit raw activations (clamp, per-channel factors) while staging
// them exist for one activation row only (the batch-1 forward, where a prep
// kernel of their own would cost a launch of its own); other batches read
// edited activations.
template <int KIND, int MB, bool BF16, int R, int XR>
static void launch_rows_xr(const RowArgs& a, int grid, int lds, hipStream_t st) {
  if constexpr (MB == 1) {
    if (a.clamp || a.xscale) return launch_rows_xe<KIND, MB, BF16, R, XR, true>(a, grid, lds, st);
  }
  launch_rows_xe<KIND, MB, BF16, R, XR, false>(a, grid, lds, st);
}

// One activation row: the first staging round is sized to the activation block
// (2, 4 or 8 slots per thread), so that short rows hold no idle staging registers.
template <int KIND, int MB, bool BF16, int R>
static hipError_t launch_rows_t(RowArgs a, int Npad, hipStream_t st) {
  const int lds = rows_lds_layout<KIND, MB>(a);
  if (lds > kRowsMaxLds || a.rank > 256)
    return hipErrorInvalidConfiguration;
  const int grid = (Npad + 4 * R - 1) / (4 * R) + a.lr_wgs;  // prologue workgroups first
  const int per_thread = (MB * a.npass * 64 * RowX<KIND>::slots + 255) / 256;
  // raw activations are edited in the first staging round only, at batch 1;
  // bf16 activations at batch 1 are staged in one round (converted to fp16 there)
  if ((a.clamp || a.xscale) && (MB != 1 || per_thread > row_x_slots1<BF16>())) return hipErrorInvalidValue;
  if (BF16 && MB == 1 && per_thread > row_x_slots1<BF16>()) return hipErrorInvalidValue;
  if constexpr (MB == 1) {
    if (per_thread <= 2)
      launch_rows_xr<KIND, MB, BF16, R, 2>(a, grid, lds, st);
    else if (per_thread <= 4)
      launch_rows_xr<KIND, MB, BF16, R, 4>(a, grid, lds, st);
    else if (per_thread <= 6)
      launch_rows_xr<KIND, MB, BF16, R, 6>(a, grid, lds, st);
    else if (!BF16 || per_thread <= 8)
      launch_rows_xr<KIND, MB, BF16, R, row_x_rounds<MB>()>(a, grid, lds, st);
    else
      launch_rows_xr<KIND, MB, BF16, R, BF16 ? 16 : row_x_rounds<MB>()>(a, grid, lds, st);
  } else {
    launch_rows_xr<KIND, MB, BF16, R, row_x_rounds<MB>()>(a, grid, lds, st);
  }
  return hipGetLastError();
}

// Whether the row-wise kernel takes this shape (its staged activations fit in
// LDS) and, in *one_round, whether it can edit raw activations: one activation
// row whose first staging round holds the whole block.
template <int KIND>
bool rows_fit(RowArgs a, bool bf16, bool* one_round = nullptr) {
  const int mb = a.M <= 1 ? 1 : a.M <= 2 ? 2 : 4;
  const int lds = mb == 1 ? rows_lds_layout<KIND, 1>(a) : mb == 2 ? rows_lds_layout<KIND, 2>(a) : rows_lds_layout<KIND, 4>(a);
  const int per_thread1 = (a.npass * 64 * RowX<KIND>::slots + 255) / 256;
  if (one_round) {  // edits: batch 1 only
    *one_round = mb == 1 && per_thread1 <= (bf16 ? row_x_slots1<true>() : row_x_slots1<false>());
  }
  // bf16 at batch 1: the whole row in one staging round
  if (bf16 && mb == 1 && per_thread1 > row_x_slots1<true>()) return false;
  return lds <= kRowsMaxLds && a.rank <= 256;
}

// Rows per wavefront: two for one activation row on layers of at least 8192
// rows (each activation chunk read from LDS serves two rows), else one, so
// that smaller layers still give every CU at least 16 wavefronts.
template <int KIND>
hipError_t launch_rows_kind(const RowArgs& a, int Npad, bool bf16, hipStream_t st) {
  if (a.M <= 1) {
    if (Npad >= 8192)
      return bf16 ? launch_rows_t<KIND, 1, true, 2>(a, Npad, st) : launch_rows_t<KIND, 1, false, 2>(a, Npad, st);
    return bf16 ? launch_rows_t<KIND, 1, true, 1>(a, Npad, st) : launch_rows_t<KIND, 1, false, 1>(a, Npad, st);
  }
  if (a.M <= 2)
    return bf16 ? launch_rows_t<KIND, 2, true, 1>(a, Npad, st) : launch_rows_t<KIND, 2, false, 1>(a, Npad, st);
  return bf16 ? launch_rows_t<KIND, 4, true, 1>(a, Npad, st) : launch_rows_t<KIND, 4, false, 1>(a, Npad, st);
}

}  // namespace cl
