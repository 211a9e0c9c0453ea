// decode_mfma.h -- batch 2..32 forward on the matrix cores, weights dequantised
// in registers.
//
// With several activation rows every weight is used M times, and the
// multiply-adds (M per weight) outgrow the vector ALUs long before the HBM
// stream does: at M = 32 a 3-bit layer needs ~7x more vector-ALU time than
// its bytes take to stream.  Here the matrix cores take the multiply-adds
// (v_mfma_f32_32x32x16, 32 weight rows x 32 activation rows x 16 k), and each
// weight is still dequantised exactly once, in the registers of the lane that
// loaded it, so the per-weight cost stays that of the batch-1 path.
//
// A workgroup of four wavefronts owns a 128-row tile and one K slice of Kz
// columns (split-K across workgroups).  Wavefront w owns rows 32w..32w+31 of
// the tile; lane l holds row 32w + (l mod 32) and, in each pass, four
// consecutive 16-byte chunks of that row (lane half h = l / 32 takes chunks
// 4h..4h+3 of the pass' eight), so every pass reads one whole 128-byte line per
// row.  The MFMA's contraction index runs over these chunks in a fixed
// permuted order: MFMA (q, j) of a pass contracts k = span*(c0 + q) + 8j..+7 on
// lane half 0 and span*(c0 + 4 + q) + 8j..+7 on half 1; the activation operand
// is read from LDS at the same k, so the sum is unchanged.
//
// 4-bit LUT tables are lane-interleaved single-entry tables (entry e of lane l
// at byte e*256 + 4l), one stacked set per wavefront, holding the values in the
// MFMA input type: every lookup is conflict-free.  3-bit LUT values stay in
// registers as byte tables and the codes are turned into values with byte
// permutes (no lookups).  The activation slice x'[0..M)[k0, k0+Kz) is staged
// once per workgroup in LDS.
//
// Outliers ("SqueezeLLM: Dense-and-Sparse Quantization", Approach: W = D + S)
// of the tile's rows inside the K slice come as per-(tile, slice, row) lists
// built when the layer is created; the two lanes of a row add them for their
// activation rows in fp32 from the staged slice.  The rank-r correction ("SLiM"
// page, review highlights: y += (x' L) R) is added by the slice-0 workgroups as
// extra MFMA steps over [t_hi | t_lo] x [R^T | R^T], t = x' L in fp32 split
// into two 16-bit parts.  t comes from the launch's first workgroups (the split
// prologue block of the batch-1 kernel, publishing the launch's generation) or
// from a kernel before it; the workgroups of the last K slice, dispatched last,
// add the rank term and wait for that generation first.  The slices' partial sums meet
// through device-scope stores, and the last workgroup of a tile adds them in
// slice order (deterministic, no float atomics).  With an activation clamp or
// per-channel activation factors the activations are edited while they are staged.
//
// Weights enter the matrix cores as 16-bit values of the activation type: fp16
// LUT values exactly for fp16 activations, rounded to nearest-even bf16 for
// bf16 activations (as on the prefill path); integer codes exactly.
#pragma once
#include <hip/hip_runtime.h>

#include "layer.h"
#include "lowrank.h"
#include "unpack.h"

namespace cl {

typedef __bf16 mf_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 mf_f16x8 __attribute__((ext_vector_type(8)));
typedef float mf_f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 mf_bf16x16 __attribute__((ext_vector_type(16)));
typedef _Float16 mf_f16x16 __attribute__((ext_vector_type(16)));
typedef uint32_t mf_u32x8 __attribute__((ext_vector_type(8)));

constexpr int kMfOe = 8;  // outlier entries per lane loaded with the code stream

struct MfArgs {
  const uint4* dense;
  const uint8_t* meta;
  const uint16_t* table;
  const void* x;
  int ldx, M, K, N, Npad, chunks;
  int tiles, S, Kz, npw;        // 128-row tiles, K slices, columns per slice, passes per slice
  const int32_t* nzs;           // bitmap: byte offset of the first kept value of every (row, slice) [Npad][S]
  uint32_t dense_bytes;         // bytes of the dense section (bitmap: the kept values)
  const int32_t* ooff;          // outlier offsets per (slice, tile, row): [S * tiles * 128 + 1]
  const uint32_t* oent;         // entries: k in slice (low 16 bits) | fp16 value << 16
  int nnz;                      // entries in oent
  const uint16_t* r16;          // R^T twice [Npad][2 rp] in the MFMA type, NULL without a rank term
  const float* t;               // t = x' L, fp32 [M][rank]
  int rank, rp;
  float* part;                  // slice partials [tiles][S][32][128]
  uint32_t* counters;           // arrivals per tile, zero between forwards
  float* y;
  int clamp;                    // clamp the activations to [-cval, cval] while staging them
  float cval;
  const uint16_t* xscale;       // then multiply them by these per-channel factors ([K] fp16; NULL: none)
  // low-rank prologue in this launch: workgroups [0, lr_wgs) run the split
  // prologue block (activation tiles of 4 rows, lr_mode 0 or 1) and publish
  // lrp.epoch (or, for epoch 0, the launch's generation), which the last
  // slice's workgroups wait for (and, in a recorded launch, count themselves
  // done after); lr_wgs = 0: t was computed by an earlier kernel
  LrSplitArgs lrp;
  int lr_wgs, lr_ntj, lr_mode;
  uint32_t lr_max_polls;  // bound of the wait for t
  uint32_t* lr_err;       // set when a wait gives up (host memory)
};

constexpr int kMfLrTile = 4;  // activation rows per tile of the prologue in this launch

template <bool BF16>
__device__ __forceinline__ mf_f32x16 mf_mfma(uint4 a, uint4 b, mf_f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(mf_bf16x8, a), __builtin_bit_cast(mf_bf16x8, b), c,
                                                   0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(mf_f16x8, a), __builtin_bit_cast(mf_f16x8, b), c, 0, 0,
                                                0);
}

// Sparse-A matrix-core step for 2:4 weights (v_smfmac_f32_32x32x32): the
// weight operand a holds eight kept values of lane (row l mod 32, half h) --
// the two kept values of each of four consecutive groups of four k -- and idx
// (bits 16 ABID ..) their 2-bit positions in the group, in the same order; the
// activation operand of lane half h' is x at 8h'..8h'+7 of lane half 0's 16 k
// (b0) and of lane half 1's (b1).  The output is transposed against mf_mfma:
// lane l holds activation row l mod 32 for weight rows 8 (v / 4) + 4 h + v mod 4.
template <bool BF16, int ABID>
__device__ __forceinline__ mf_f32x16 mf_smfmac(uint4 a, uint4 b0, uint4 b1, uint32_t idx, mf_f32x16 c) {
  const mf_u32x8 b = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  if constexpr (BF16)
    return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(mf_bf16x8, a), __builtin_bit_cast(mf_bf16x16, b), c,
                                                     (int)idx, 0, ABID);
  return __builtin_amdgcn_smfmac_f32_32x32x32_f16(__builtin_bit_cast(mf_f16x8, a), __builtin_bit_cast(mf_f16x16, b), c,
                                                  (int)idx, 0, ABID);
}

template <bool BF16>
__device__ __forceinline__ uint32_t mf_to16(float f) {
  if constexpr (BF16) return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

template <bool BF16>
__device__ __forceinline__ float mf_act(uint32_t v16) {
  if constexpr (BF16) return __uint_as_float(v16 << 16);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)v16);
}

// A VGPR holding a constant, so that (x & c) | sgpr folds into one v_and_or_b32
// (a VOP3 instruction takes one scalar or literal operand on this target).
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(c));
  return v;
}

// Two 16-bit table values into one register: the first into the low half
// (ds_read_u16_d16), the second into the high half (ds_read_u16_d16_hi).
__device__ __forceinline__ uint32_t lds_pair16(const uint32_t* lds, uint32_t a_lo, uint32_t a_hi) {
  half2_t r;
  r.x = *reinterpret_cast<const _Float16*>(reinterpret_cast<const uint8_t*>(lds) + a_lo);
  r.y = *reinterpret_cast<const _Float16*>(reinterpret_cast<const uint8_t*>(lds) + a_hi);
  return as_u32(r);
}

// 4-bit LUT word (device byte order: the pair (c_2b, c_2b+1) rotated left by
// two bits in byte b) through lane-interleaved single-entry tables: four pairs.
__device__ __forceinline__ void lut4_word_single(const uint32_t* lds, uint32_t w, uint32_t lanebase, uint32_t out[4],
                                                 uint32_t b, uint32_t m15, uint32_t m3, uint32_t m12) {
  const uint32_t ev = ((w >> 2) & m15) | b;                            // bits 2..5: c_2b
  const uint32_t od = ((w >> 6) & m3) | ((w << 2) & m12) | b;          // bits 6..7, 0..1: c_2b+1
  out[0] = lds_pair16(lds, addr_from_byte<0>(ev, lanebase), addr_from_byte<0>(od, lanebase));
  out[1] = lds_pair16(lds, addr_from_byte<1>(ev, lanebase), addr_from_byte<1>(od, lanebase));
  out[2] = lds_pair16(lds, addr_from_byte<2>(ev, lanebase), addr_from_byte<2>(od, lanebase));
  out[3] = lds_pair16(lds, addr_from_byte<3>(ev, lanebase), addr_from_byte<3>(od, lanebase));
}

// MT = activation rows staged.  The 4-bit LUT uses lane-interleaved
// single-entry tables: one lookup per weight, but conflict-free.  (3-bit LUT
// single-entry lookups, with an address permute per value and a permute per
// pair, cost more vector issue than byte permutes over the values held in
// registers, and they were replaced by those.  Per-row pair tables, one
// lookup per two weights, measured slower here: the 32 rows of a wavefront
// look up different tables, and their bank conflicts cost more than the
// lookups they save.)
//
// The bitmap format takes one 128-k chunk per lane half and pass: its kept
// values sit at data-dependent offsets, so each lane stages the window holding
// its chunk's kept bytes (at most 144 bytes from a 16-byte aligned start) in a
// slot of its own in LDS, and expands it by the chunk's keep bits with the
// nibble selector table (the tile kernel's expansion).
constexpr int kMfBmSlot = 37;  // dwords per lane slot (odd: lanes fall in distinct banks)
template <int KIND, int MT>
struct MfCfg {
  static constexpr int span = KindTraits<KIND>::span, pairs = KindTraits<KIND>::pairs;
  static constexpr int cph = KIND == K_INT8_BM ? 1 : kMfCph;  // chunks per lane half per pass
  static constexpr int passk = 2 * cph * span;                // k per pass
  static constexpr int ents = KIND == K_LUT4 ? 16 : 0;  // LDS table entries per row (LUT3: values in registers)
  // static LDS at address 0: four stacked lane-interleaved single-entry table
  // sets, the 2:4 selectors, or the bitmap's nibble selectors and lane slots
  static constexpr int tab_bytes = ents ? 4 * ents * 256
                                   : KIND == K_INT4_24 ? 128
                                   : KIND == K_INT8_BM ? (kBmSelDwords + 256 * kMfBmSlot) * 4
                                                       : 16;
  static constexpr int ok_word = tab_bytes / 4;  // after the tables: whether t was published
};

// LDS bytes per staged activation row: the slice padded so that the row
// stride is 16 mod 256 bytes (16-byte reads of 16 consecutive rows are
// conflict-free).
__host__ __device__ inline int mf_xrow(int Kz) { return ((Kz * 2 + 255) / 256) * 256 + 16; }
__host__ __device__ inline int mf_trow(int rp) { return ((4 * rp + 255) / 256) * 256 + 16; }

// MT = activation rows staged (M <= MT).
template <int KIND, bool BF16, int MT>
__global__ void __launch_bounds__(256, 2) decode_mfma_kernel(MfArgs a) {
  using C = MfCfg<KIND, MT>;
  constexpr int SPAN = C::span, P = C::pairs, PASSK = C::passk, NMF = P / 4;  // MFMAs per chunk
  constexpr int CPH = C::cph;
  constexpr bool BM = KIND == K_INT8_BM;
  constexpr bool SP = KIND == K_INT4_24;  // 2:4 on the sparse-A instruction (kept values and positions as stored)
  // outputs v of a lane whose activation row m(v) = 8 (v / 4) + 4 half + v mod 4 is below MT
  constexpr int NV = MT >= 32 ? 16 : MT / 2;
  constexpr int XR = MT * kMfKzMax / 8 / 256;  // 16-byte activation slots per thread
  constexpr bool LUT = KIND == K_LUT3 || KIND == K_LUT4;
  __shared__ __attribute__((aligned(16))) uint32_t stab[C::tab_bytes / 4 + 4];  // at LDS address 0
  extern __shared__ __attribute__((aligned(16))) uint32_t sdyn[];          // activation slice, then t

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (a.lr_wgs > 0 && (int)blockIdx.x < a.lr_wgs) {  // a prologue workgroup
    const int b = blockIdx.x, S = a.lrp.S, s = b % S, tj = (b / S) % a.lr_ntj, tm = b / (S * a.lr_ntj);
    uint8_t* smem = reinterpret_cast<uint8_t*>(sdyn);
    if (a.lr_mode == 0) lr_split_block<0, kMfLrTile, BF16, true>(a.lrp, s, tj, tm, a.lr_ntj, smem);
    else lr_split_block<1, kMfLrTile, BF16, true>(a.lrp, s, tj, tm, a.lr_ntj, smem);
    return;
  }
  const int bid = (int)blockIdx.x - a.lr_wgs;
  const int tile = bid % a.tiles, z = bid / a.tiles;
  const int rt = wave * 32 + (lane & 31);  // row in tile
  const int n = tile * kMfRows + rt;       // weight row of this lane (>= Npad: reads zeros)
  const int k0 = z * a.Kz;
  const int xrow = mf_xrow(a.Kz);
  uint8_t* sb = reinterpret_cast<uint8_t*>(sdyn);

  // ---- outlier range of this lane's (slice, tile, row) ----
  const int vr = (z * a.tiles + tile) * kMfRows + rt;
  const bool has_csr = a.ooff != nullptr;
  int oe0 = 0, oe1 = 0;
  if (has_csr) {
    const brsrc_t ro = make_rsrc(a.ooff, (uint32_t)(a.S * a.tiles * kMfRows + 1) * 4u);
    oe0 = (int)bload32(ro, (uint32_t)vr * 4u, 0);
    oe1 = (int)bload32(ro, (uint32_t)(vr + 1) * 4u, 0);
  }

  // ---- LUT values or row scale of this lane's row ----
  constexpr uint32_t TBYTES = KIND == K_LUT4 ? 32u : KIND == K_LUT3 ? 16u : 2u;
  const brsrc_t rtab = make_rsrc(a.table, (uint32_t)a.Npad * TBYTES);
  uint4 tv0 = make_uint4(0, 0, 0, 0), tv1 = make_uint4(0, 0, 0, 0);
  uint32_t scale16 = 0;
  if constexpr (LUT) {
    tv0 = bload128(rtab, (uint32_t)n * TBYTES, 0);
    if constexpr (KIND == K_LUT4) tv1 = bload128(rtab, (uint32_t)n * TBYTES + 16u, 0);
  } else {
    scale16 = bload16(rtab, (uint32_t)n * 2u, 0);
  }

  // ---- activation slice (rows >= M and columns >= ldx read zero) ----
  const int slots_row = a.Kz / 8;
  const brsrc_t rx = make_rsrc(a.x, (uint32_t)a.M * (uint32_t)a.ldx * 2u);
  uint4 xs[XR];
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int s = i * 256 + tid, m = s / slots_row, c = s - m * slots_row, k = k0 + 8 * c;
    const bool ok = m < a.M && k < a.ldx;
    xs[i] = bload128(rx, ok ? ((uint32_t)m * (uint32_t)a.ldx + (uint32_t)k) * 2u : kNoLoad, 0);
  }
  if (a.xscale) {
    // clamped and scaled before the code stream is issued (one exposed load
    // latency), so that the factors hold no registers while it is in flight
    const brsrc_t rf = make_rsrc(a.xscale, (uint32_t)a.ldx * 2u);
    uint4 xf[XR];
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int s = i * 256 + tid, m = s / slots_row, c = s - m * slots_row, k = k0 + 8 * c;
      xf[i] = bload128(rf, m < a.M && k < a.ldx ? (uint32_t)k * 2u : kNoLoad, 0);
    }
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      if (a.clamp) xs[i] = clamp_act8<BF16>(xs[i], a.cval);
      xs[i] = scale_act8<BF16>(xs[i], xf[i]);
    }
  }

  __builtin_amdgcn_sched_barrier(0);
  // ---- the code stream: passes of four chunks per lane, three in flight ----
  const int cbase = k0 / SPAN;  // first chunk of the slice (Kz is a whole number of passes)
  const brsrc_t rd = make_rsrc(a.dense, (uint32_t)a.Npad * (uint32_t)a.chunks * 16u);
  const brsrc_t rm = make_rsrc(a.meta, KIND == K_INT4_24 ? (uint32_t)a.Npad * (uint32_t)a.chunks * 8u : 0u);
  auto load_pass = [&](uint4 (&w)[CPH], uint2 (&mw)[CPH], int p) {
#pragma unroll
    for (int q = 0; q < CPH; ++q) {
      const int c = cbase + p * 2 * CPH + half * CPH + q;
      const bool ok = p < a.npw && c < a.chunks;
      const uint32_t idx = (uint32_t)n * (uint32_t)a.chunks + (uint32_t)c;
      w[q] = bload128_nt(rd, ok ? idx * 16u : kNoLoad, 0);
      if constexpr (KIND == K_INT4_24)
        mw[q] = bload64_nt(rm, ok ? idx * 8u : kNoLoad, 0);
      else
        mw[q] = make_uint2(0, 0);
    }
  };
  uint4 WA[CPH], WB[CPH], WC[CPH];
  uint2 MA[CPH], MB[CPH], MC[CPH];
  // bitmap: the keep bits of every pass of the slice and the slice's first kept byte
  constexpr int NPB = kMfKzMax / (BM ? PASSK : kMfKzMax);
  uint4 bmeta[NPB];
  uint32_t nz0 = 0;
  if constexpr (BM) {
#pragma unroll
    for (int p = 0; p < NPB; ++p) {
      const int c = cbase + 2 * p + half;
      const bool ok = p < a.npw && c < a.chunks;
      bmeta[p] = bload128(make_rsrc(a.meta, (uint32_t)a.Npad * (uint32_t)a.chunks * 16u),
                          ok ? ((uint32_t)n * (uint32_t)a.chunks + (uint32_t)c) * 16u : kNoLoad, 0);
    }
    nz0 = bload32(make_rsrc(a.nzs, (uint32_t)a.Npad * (uint32_t)a.S * 4u), ((uint32_t)n * (uint32_t)a.S + (uint32_t)z) * 4u, 0);
  } else {
    load_pass(WA, MA, 0);
    load_pass(WB, MB, 1);
    load_pass(WC, MC, 2);
  }
  // keep the issue order (the outlier entries below wait for their offsets:
  // issued before the code stream they would hold it back by one latency)
  __builtin_amdgcn_sched_barrier(0);

  // ---- the first kMfOe outlier entries of this lane's list (consumed at the end) ----
  uint32_t oent[kMfOe];
  {
    const brsrc_t re = make_rsrc(a.oent, has_csr ? (uint32_t)a.nnz * 4u : 0u);  // uniform: no waterfall loop
#pragma unroll
    for (int i = 0; i < kMfOe; ++i) oent[i] = bload32(re, oe0 + i < oe1 ? (uint32_t)(oe0 + i) * 4u : kNoLoad, 0);
  }

  // ---- LDS: activation slice (rows M..MT-1 zero) plus a zero row MT, tables ----
  if (a.clamp && !a.xscale) {
#pragma unroll
    for (int i = 0; i < XR; ++i) xs[i] = clamp_act8<BF16>(xs[i], a.cval);
  }
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int s = i * 256 + tid, m = s / slots_row, c = s - m * slots_row;
    if (m < MT && s < MT * slots_row)
      *reinterpret_cast<uint4*>(sb + m * xrow + c * 16) = xs[i];
  }
  for (int c = tid; c < slots_row; c += 256) *reinterpret_cast<uint4*>(sb + MT * xrow + c * 16) = make_uint4(0, 0, 0, 0);
  const uint32_t lanebase = (uint32_t)lane * 4u, ebias = (uint32_t)(wave * C::ents);
  auto lut_val = [&](uint32_t h) -> uint32_t {
    return BF16 ? mf_to16<true>((float)__builtin_bit_cast(_Float16, (uint16_t)h)) : h;
  };
  if constexpr (KIND == K_LUT4) {
    const uint32_t lw[8] = {tv0.x, tv0.y, tv0.z, tv0.w, tv1.x, tv1.y, tv1.z, tv1.w};
#pragma unroll
    for (int e = 0; e < C::ents; ++e) {
      const uint32_t h = (lw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      stab[(ebias + e) * 64 + lane] = lut_val(h);
    }
  } else if constexpr (KIND == K_INT4_24) {
    if (tid < 16) {
      const uint2 e = seltab_2_4_entry((uint32_t)tid);
      stab[2 * tid] = e.x;
      stab[2 * tid + 1] = e.y;
    }
  } else if constexpr (BM) {
    if (tid < 16) stab[tid] = bitmap_sel_entry((uint32_t)tid);
  }
  __syncthreads();

  // ---- dequantise, multiply on the matrix cores ----
  mf_f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  const int mrow = lane & 31;  // activation row of this lane's A operand
  // mask constants in VGPRs and the table-set bias in every byte
  const uint32_t bias4 = ebias * 0x01010101u;
  Lut3Bytes T3 = {0, 0, 0, 0};  // LUT3: the row's values as byte tables in registers
  if constexpr (KIND == K_LUT3) T3 = lut3_bytes<BF16>(tv0);
  uint32_t mk0 = 0, mk1 = 0, mk2 = 0;
  if constexpr (KIND == K_LUT4) {
    mk0 = vconst(0x0F0F0F0Fu);
    mk1 = vconst(0x03030303u);
    mk2 = vconst(0x0C0C0C0Cu);
  }
  const int mrow_s = mrow < MT ? mrow : MT;  // rows past MT read the zero row
  const uint8_t* xr = sb + mrow_s * xrow + half * CPH * SPAN * 2;
  const uint8_t* xsp = sb + mrow_s * xrow + half * 16;  // 2:4: lane half h' reads k 8h'..8h'+7 of each 16-k segment
  if constexpr (BM) {
    // kept-byte windows: lane half h's chunk of pass p starts after the slice's
    // earlier kept values and, for h = 1, after its partner's (lane l - 32) chunk
    uint32_t start[NPB], cnt[NPB];
    {
      uint32_t run = nz0;
#pragma unroll
      for (int p = 0; p < NPB; ++p) {
        cnt[p] = __builtin_popcount(bmeta[p].x) + __builtin_popcount(bmeta[p].y) + __builtin_popcount(bmeta[p].z) +
                 __builtin_popcount(bmeta[p].w);
        const uint32_t pc = (uint32_t)__shfl_xor((int)cnt[p], 32, 64);
        start[p] = run + (half ? pc : 0u);
        run += cnt[p] + pc;
      }
    }
    const brsrc_t rk = make_rsrc(a.dense, a.dense_bytes);  // kept values; a window past the end reads zero
    auto load_kept = [&](uint4 (&kw)[9], int p) {
      const uint32_t b0 = start[p < NPB ? p : 0] & ~15u, end = start[p < NPB ? p : 0] + cnt[p < NPB ? p : 0];
#pragma unroll
      for (int i = 0; i < 9; ++i) kw[i] = bload128(rk, p < a.npw && b0 + 16u * i < end ? b0 + 16u * i : kNoLoad, 0);
    };
    uint4 KA[9], KB[9];
    load_kept(KA, 0);
    load_kept(KB, 1);
    const uint32_t slot = (uint32_t)(kBmSelDwords + tid * kMfBmSlot) * 4u;
    auto comp_bm = [&](const uint4 (&kw)[9], int p) {
      if (p >= a.npw) return;
      uint32_t* sl = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(stab) + slot);
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        sl[4 * i] = kw[i].x;
        sl[4 * i + 1] = kw[i].y;
        sl[4 * i + 2] = kw[i].z;
        sl[4 * i + 3] = kw[i].w;
      }
      uint32_t off = slot + (start[p] & 15u);
      const uint32_t mw4[4] = {bmeta[p].x, bmeta[p].y, bmeta[p].z, bmeta[p].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // 32 k of the chunk
        uint32_t wp[16];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint32_t nib = (mw4[i] >> (4 * t)) & 0xFu;
          const uint32_t lo = lds_u32(stab, off & ~3u), hi = lds_u32(stab, (off & ~3u) + 4u);
          const uint32_t win = __builtin_amdgcn_alignbyte(hi, lo, off & 3u);
          int8x4_signed(perm(0u, win, lds_u32(stab, nib * 4u)), &wp[2 * t]);
          off += __builtin_popcount(nib);
        }
        if constexpr (BF16) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const half2_t hv = as_h2(wp[j]);
            wp[j] = mf_to16<true>((float)hv.x) | (mf_to16<true>((float)hv.y) << 16);
          }
        }
        const uint8_t* xq = xr + (p * PASSK + 32 * i) * 2;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 xa = *reinterpret_cast<const uint4*>(xq + 16 * j);
          acc = mf_mfma<BF16>(xa, make_uint4(wp[4 * j], wp[4 * j + 1], wp[4 * j + 2], wp[4 * j + 3]), acc);
        }
      }
    };
#pragma unroll
    for (int p = 0; p < NPB; p += 2) {
      comp_bm(KA, p);
      load_kept(KA, p + 2);
      comp_bm(KB, p + 1);
      load_kept(KB, p + 3);
    }
  } else {
  auto comp_pass = [&](const uint4 (&w)[CPH], const uint2 (&mw)[CPH], int p) {
    if (p >= a.npw) return;
#pragma unroll
    for (int q = 0; q < CPH; ++q) {
      const uint32_t ww[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
      if constexpr (SP) {
        // word i of the chunk holds the kept pairs of groups 4i..4i+3 (16 k of
        // the row) and meta bits 16 (i mod 2).. of word i / 2 their positions:
        // one sparse step per word, lane half 1 on the chunk four later
        const uint8_t* x0 = xsp + (p * PASSK + q * SPAN) * 2;
        const uint8_t* x1 = xsp + (p * PASSK + (CPH + q) * SPAN) * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t v[4];
          int4_word(ww[i], v);
          if constexpr (BF16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const half2_t hv = as_h2(v[j]);
              v[j] = mf_to16<true>((float)hv.x) | (mf_to16<true>((float)hv.y) << 16);
            }
          }
          const uint4 av = make_uint4(v[0], v[1], v[2], v[3]);
          const uint4 b0 = *reinterpret_cast<const uint4*>(x0 + 32 * i);
          const uint4 b1 = *reinterpret_cast<const uint4*>(x1 + 32 * i);
          const uint32_t idx = i < 2 ? mw[q].x : mw[q].y;
          acc = (i & 1) ? mf_smfmac<BF16, 1>(av, b0, b1, idx, acc) : mf_smfmac<BF16, 0>(av, b0, b1, idx, acc);
        }
        continue;
      }
      uint32_t wp[P];
      if constexpr (KIND == K_LUT3) {
#pragma unroll
        for (int i = 0; i < 4; ++i) lut3_word_perm(ww[i], T3, &wp[5 * i]);
      } else if constexpr (KIND == K_LUT4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) lut4_word_single(stab, ww[i], lanebase, &wp[4 * i], bias4, mk0, mk1, mk2);
      } else {
        chunk_pairs<KIND, false>(stab, w[q], make_uint4(mw[q].x, mw[q].y, 0, 0), lanebase, 0u, wp, ebias);
        if constexpr (!LUT && BF16) {
#pragma unroll
          for (int j = 0; j < P; ++j) {
            const half2_t hv = as_h2(wp[j]);
            wp[j] = mf_to16<true>((float)hv.x) | (mf_to16<true>((float)hv.y) << 16);
          }
        }
      }
      const uint8_t* xq = xr + (p * PASSK + q * SPAN) * 2;
#pragma unroll
      for (int j = 0; j < NMF; ++j) {
        const uint4 xa = *reinterpret_cast<const uint4*>(xq + 16 * j);
        acc = mf_mfma<BF16>(xa, make_uint4(wp[4 * j], wp[4 * j + 1], wp[4 * j + 2], wp[4 * j + 3]), acc);
      }
    }
  };
  // three passes in flight; the first three outside the loop, so that their waits are exact
  comp_pass(WA, MA, 0);
  load_pass(WA, MA, 3);
  comp_pass(WB, MB, 1);
  load_pass(WB, MB, 4);
  comp_pass(WC, MC, 2);
  load_pass(WC, MC, 5);
  for (int p = 3; p < a.npw; p += 3) {
    comp_pass(WA, MA, p);
    load_pass(WA, MA, p + 3);
    comp_pass(WB, MB, p + 1);
    load_pass(WB, MB, p + 4);
    comp_pass(WC, MC, p + 2);
    load_pass(WC, MC, p + 5);
  }

  }
  // lane l holds row rt for activation rows m(v) = 8 (v / 4) + 4 half + v mod 4
  // (2:4: transposed, brought back below, after the outliers)
  const mf_f32x16 dsum = acc;
  // ---- integer formats: the row scale multiplies the dense part only ----
  const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)scale16);
  if constexpr (SP) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  } else if constexpr (!LUT) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] *= sc;
  }
  // ---- outliers of this row inside the slice, activations from the staged
  // slice (rows M..MT-1 are zero there, so no batch test is needed) ----
  if (has_csr) {
    const brsrc_t re = make_rsrc(a.oent, (uint32_t)a.nnz * 4u);
    uint32_t moff[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) moff[v] = (uint32_t)((8 * (v >> 2) + 4 * half + (v & 3)) * xrow);
    for (int e = oe0; e < oe1; ++e) {
      const int i = e - oe0;
      uint32_t en = oent[0];
#pragma unroll
      for (int u = 1; u < kMfOe; ++u)
        if (i == u) en = oent[u];
      if (i >= kMfOe) en = bload32(re, (uint32_t)e * 4u, 0);  // lists longer than the prefetch
      const uint32_t kk2 = (en & 0xFFFFu) * 2u;
      const float val = (float)__builtin_bit_cast(_Float16, (uint16_t)(en >> 16));
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[v] = __builtin_fmaf(val, mf_act<BF16>(lds_u16(sdyn, moff[v] + kk2)), acc[v]);
    }
  }
  if constexpr (SP) {
    // the dense sums to this lane's row through LDS (each wave's own 32 x 33
    // floats of the activation slice's space, free once every wave is past
    // the outliers), times the row scale, plus the outliers
    __syncthreads();
    float* tr = reinterpret_cast<float*>(sb) + wave * (32 * 33);
#pragma unroll
    for (int v = 0; v < 16; ++v) tr[(8 * (v >> 2) + 4 * half + (v & 3)) * 33 + (lane & 31)] = dsum[v];
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = __builtin_fmaf(tr[(lane & 31) * 33 + 8 * (v >> 2) + 4 * half + (v & 3)], sc, acc[v]);
    __syncthreads();  // the space is reused below (t, the last-arrival flag)
  }
  // ---- rank term (last slice): [t_hi | t_lo] x [R^T | R^T] on the matrix cores ----
  if (a.r16 != nullptr && z == a.S - 1) {
    const int rp2 = 2 * a.rp, trow = mf_trow(a.rp);
    const uint32_t target = a.lr_wgs > 0 ? lr_target(a.lrp.flag, a.lrp.epoch) : 0u;
    if (wave == 0) {
      const bool ok = a.lr_wgs == 0 ||
                      wait_lowrank(lr_word(a.lrp.flag, a.lrp.epoch), target, lane, a.lr_max_polls, a.lr_err);
      if (lane == 0) stab[C::ok_word] = ok ? 1u : 0u;
    }
    __syncthreads();  // t is published (or the wait gave up); every wave is done with the activation slice
    const bool t_ok = stab[C::ok_word] != 0u;
    for (int i = tid; i < (MT + 1) * a.rp; i += 256) {  // row MT: zeros
      const int m = i / a.rp, j = i - m * a.rp;
      const float tv = (m < a.M && j < a.rank) ? (t_ok ? load_dev(a.t + (size_t)m * a.rank + j) : __builtin_nanf("")) : 0.f;
      const uint32_t hi = mf_to16<BF16>(tv);
      const float hf = BF16 ? __uint_as_float(hi << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)hi);
      const uint32_t lo = mf_to16<BF16>(tv - hf);
      *reinterpret_cast<uint16_t*>(sb + m * trow + j * 2) = (uint16_t)hi;
      *reinterpret_cast<uint16_t*>(sb + m * trow + (a.rp + j) * 2) = (uint16_t)lo;
    }
    __syncthreads();  // the workgroup's reads of t are done (their values are in LDS)
    if (a.lr_wgs > 0 && a.lrp.epoch == 0 && tid == 0) lr_reader_done(a.lrp.flag, target, a.tiles, tile);
    const brsrc_t rr = make_rsrc(a.r16, (uint32_t)a.Npad * (uint32_t)rp2 * 2u);
    for (int s = 0; s < rp2 / 16; ++s) {
      const uint4 wv = bload128(rr, ((uint32_t)n * (uint32_t)rp2 + (uint32_t)(16 * s + 8 * half)) * 2u, 0);
      const uint4 ta = *reinterpret_cast<const uint4*>(sb + mrow_s * trow + (16 * s + 8 * half) * 2);
      acc = mf_mfma<BF16>(ta, wv, acc);
    }
  }

  // ---- store, or combine the slices' partial sums (last workgroup of the tile) ----
  if (a.S == 1) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 8 * (v >> 2) + 4 * half + (v & 3);
      if (m < a.M && n < a.N) a.y[(size_t)m * a.N + n] = acc[v];
    }
    return;
  }
  // Partial sums cross workgroups (possibly on different XCDs, whose L2s are
  // not coherent with each other) through device-scope stores and loads.
  float* mypart = a.part + ((size_t)tile * a.S + z) * (32 * kMfRows);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int m = 8 * (v >> 2) + 4 * half + (v & 3);
    if (m < a.M) store_dev(mypart + m * kMfRows + rt, acc[v]);
  }
  wait_stores();
  __syncthreads();  // every wave is past its last read of the staged slice: its first dword holds the flag
  // LDS-typed: a generic volatile pointer would be a flat access, waited for with every memory operation
  volatile __attribute__((address_space(3))) uint32_t* s_last =
      reinterpret_cast<volatile __attribute__((address_space(3))) uint32_t*>(reinterpret_cast<uintptr_t>(sdyn));
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_last = old == (uint32_t)(a.S - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!*s_last) return;
  // each thread owns outputs (m, row) tid + 256 o; per round of eight outputs
  // and group of eight slices all 64 loads are issued before any is added, so
  // the reduction waits about S / 8 latencies per round, not S
  const float* tp = a.part + (size_t)tile * a.S * (32 * kMfRows);
  const int nout = a.M * kMfRows;
  for (int ob = 0; ob < nout; ob += 8 * 256) {
    float acc_o[8];
#pragma unroll
    for (int o = 0; o < 8; ++o) acc_o[o] = 0.f;
    for (int s0 = 0; s0 < a.S; s0 += 8) {
      float v8[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int o = 0; o < 8; ++o) {
          const int i = ob + tid + 256 * o;
          v8[u][o] = (s0 + u < a.S && i < nout) ? load_dev(tp + (size_t)(s0 + u) * (32 * kMfRows) + i) : 0.f;
        }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int o = 0; o < 8; ++o) acc_o[o] += v8[u][o];  // slices in order for every output
    }
#pragma unroll
    for (int o = 0; o < 8; ++o) {
      const int i = ob + tid + 256 * o, m = i / kMfRows, row = tile * kMfRows + (i - m * kMfRows);
      if (i < nout && row < a.N) a.y[(size_t)m * a.N + row] = acc_o[o];
    }
  }
  if (tid == 0) __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next forward
}

template <int KIND, bool BF16, int MT>
static hipError_t launch_mfma_t(const MfArgs& a, hipStream_t st) {
  const int lds_x = (MT + 1) * mf_xrow(a.Kz);
  const int lds_t = a.r16 ? (MT + 1) * mf_trow(a.rp) : 0;
  const int lds_l = a.lr_wgs > 0 ? lr_scratch_bytes(a.lr_mode, kMfLrTile) : 0;  // prologue workgroups
  int lds = lds_x > lds_t ? lds_x : lds_t;
  lds = lds > lds_l ? lds : lds_l;
  if constexpr (KIND == K_INT4_24) lds = lds > 4 * 32 * 33 * 4 ? lds : 4 * 32 * 33 * 4;  // the 2:4 transposition
  hipLaunchKernelGGL((decode_mfma_kernel<KIND, BF16, MT>), dim3(a.lr_wgs + a.tiles * a.S), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_mfma_kind(const MfArgs& a, bool bf16, hipStream_t st) {
  if (a.Kz > kMfKzMax || a.Kz % MfCfg<KIND, 32>::passk || a.M > 32 || a.M < 1 || a.Kz >= 65536)
    return hipErrorInvalidValue;
  if (a.M <= 8) return bf16 ? launch_mfma_t<KIND, true, 8>(a, st) : launch_mfma_t<KIND, false, 8>(a, st);
  if (a.M <= 16) return bf16 ? launch_mfma_t<KIND, true, 16>(a, st) : launch_mfma_t<KIND, false, 16>(a, st);
  return bf16 ? launch_mfma_t<KIND, true, 32>(a, st) : launch_mfma_t<KIND, false, 32>(a, st);
}

}  // namespace cl
