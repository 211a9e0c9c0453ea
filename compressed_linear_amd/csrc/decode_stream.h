// decode_stream.h -- batch-1 forward streamed by resident wavefronts.
//
// The row-wise kernel gives each wavefront two rows: every wavefront issues
// its loads, waits, then multiplies, so the memory latency and the vector work
// of the resident wavefronts follow each other instead of overlapping, and the
// per-workgroup work (staging the activations) is spread over only eight rows.
// Here a workgroup of 4..8 wavefronts owns a contiguous range of rows sized so
// that all workgroups are resident at once (two per CU), and each wavefront
// walks its own rows two at a time ("groups") with the code stream pipelined
// across group boundaries: while one group is multiplied, the codes of the
// next ones are in flight.
//
// Everything a group needs besides its codes is staged in LDS once per
// workgroup before the walk (the activations, converted to fp16 with a row
// scale when they are bf16; the LUT values or row scales, row pointers and
// rank-factor rows of the workgroup's rows) or once per wavefront (the
// outliers of its rows, packed as column | fp16 value << 16), so the loads
// inside the walk are the code blocks alone and the compiler's load counting
// stays exact.  Dequantisation, the balanced outlier spread over the lanes
// ("SqueezeLLM: Dense-and-Sparse Quantization", Approach and measured-effects
// table) and the rank-r term ("SLiM" page, review highlights) are those of the
// row-wise kernel; t = x' L_hat comes from the launch's first workgroups.
#pragma once
#include <hip/hip_runtime.h>

#include "decode_rows.h"

namespace cl {

constexpr int kStMaxWaves = 8;    // wavefronts per workgroup (4..8)
constexpr int kStOutLoads = 8;    // outlier entries a lane loads for its wavefront
constexpr int kStMaxRows = 128;   // rows per workgroup (metadata staged one vector per thread)
constexpr int kStRankBytes = 8192;  // rank-factor bytes staged per workgroup (two vectors per thread)

struct StreamArgs {
  RowArgs r;            // pointers, sizes, activation edits, the in-launch prologue
  int rows_per_wg;      // RW: rows of each workgroup (a multiple of 8)
  int npass;            // passes of 64 chunks per row
  int lds_meta;         // LDS byte offsets: per-row LUT values / scales,
  int lds_rp;           //   row pointers (RW + 1),
  int lds_rank;         //   rank-factor rows (RW x rank_row_bytes),
  int lds_rsc;          //   int4 rank-factor scales (RW x rsc_row_bytes),
  int lds_out;          //   outliers, out_cap entries per wavefront
  int rank_row_bytes;   // bytes of one R^T row (16-bit: 2 rank, int4: ceil(rank / 2))
  int rsc_row_bytes;    // bytes of one row of int4 R^T scales
  int out_cap;          // outlier entries staged per wavefront (<= 64 * kStOutLoads)
  int row_waves;        // wavefronts of the row workgroups (readers of t in a recorded launch)
};

__device__ __forceinline__ float wave_sum_dpp(float v) {
  // rows of 16 lanes: quad swaps, then rotations by 4 and 8; then the four rows in a fixed order
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// NB = passes per block of the code stream (two blocks in flight), XR =
// activation slots staged per thread (one round), LR = low-rank part, EDIT =
// raw activations edited (clamp, per-channel factors) while staged.
template <int KIND, bool BF16, int NB, int XR, bool LR, bool EDIT>
__global__ void __launch_bounds__(512) decode_stream_kernel(StreamArgs sa) {
  const RowArgs& a = sa.r;
  constexpr int R = 2;
  constexpr int SPAN = KindTraits<KIND>::span, P = KindTraits<KIND>::pairs, XD = SPAN / 8;
  constexpr int XS = RowX<KIND>::stride, XSL = RowX<KIND>::slots;
  constexpr bool LUT = KIND == K_LUT3 || KIND == K_LUT4;
  constexpr uint32_t RTB = (uint32_t)row_table_bytes<KIND>();
  constexpr uint32_t TB = KIND == K_LUT4 ? 32u : KIND == K_LUT3 ? 16u : 2u;  // metadata bytes per row
  constexpr int TABW = LUT ? kStMaxWaves * R * (int)RTB / 4 : (KIND == K_INT4_24 ? 64 : 4);
  __shared__ __attribute__((aligned(16))) uint32_t stab[TABW + kStMaxWaves];  // tables at LDS address 0, then row maxima
  extern __shared__ __attribute__((aligned(16))) uint32_t sdyn[];
  uint8_t* sb = reinterpret_cast<uint8_t*>(sdyn);
  const int tid = threadIdx.x, nthr = blockDim.x, wpg = nthr >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  if constexpr (LR) {
    if ((int)blockIdx.x < a.lr_wgs) {  // a prologue workgroup (threads past 256 only keep the barriers)
      const int b = blockIdx.x, S = a.lrp.S, s = b % S, tj = (b / S) % a.lr_ntj, tm = b / (S * a.lr_ntj);
      if (a.lr_mode == 0) lr_split_block<0, 1, BF16, EDIT>(a.lrp, s, tj, tm, a.lr_ntj, sb);
      else lr_split_block<1, 1, BF16, EDIT>(a.lrp, s, tj, tm, a.lr_ntj, sb);
      return;
    }
  }
  const int wg = (int)blockIdx.x - (LR ? a.lr_wgs : 0);
  const int r0 = wg * sa.rows_per_wg;                       // first row of the workgroup
  const int rw = min(sa.rows_per_wg, a.N - r0);             // its rows (>= 1)
  const int ngr = (rw + R - 1) / R;                         // its groups
  const int nq = (ngr + wpg - 1) / wpg;                     // groups per wavefront
  const int q0 = wave * nq, nqw = max(0, min(q0 + nq, ngr) - q0);  // this wavefront's groups [q0, q0 + nqw)
  const bool has_csr = a.rowptr != nullptr;

  // ---- activations: one staging round (XR slots per thread) ----
  const int SM = sa.npass * 64 * XSL;  // slots of the row
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
    for (int i = 0; i < XR; ++i) xf[i] = a.xscale ? bload128(rf, x_src(i * nthr + tid), 0) : make_uint4(0, 0, 0, 0);
  }

  // ---- metadata of the workgroup's rows (one or two vectors per thread) ----
  const brsrc_t rtab = make_rsrc(a.table, (uint32_t)a.Npad * TB);
  const uint32_t mbytes = (uint32_t)rw * TB;
  const uint4 mv = bload128(rtab, (uint32_t)(16 * tid) < mbytes ? (uint32_t)r0 * TB + 16u * (uint32_t)tid : kNoLoad, 0);
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

  // ---- the code stream: blocks of NB passes of this wavefront's groups, two in flight ----
  const int nblk = (sa.npass + NB - 1) / NB, TBK = nqw * nblk;
  const brsrc_t rd = make_rsrc(a.dense, (uint32_t)a.Npad * (uint32_t)a.chunks * 16u);
  const brsrc_t rm = make_rsrc(a.meta, KIND == K_INT4_24 ? (uint32_t)a.Npad * (uint32_t)a.chunks * 8u : 0u);
  int lq = 0, lbb = 0;  // group and block of the next load
  auto load_blk = [&](uint4 (&w)[NB][R], uint2 (&mw)[NB][R], int j) {
    const int n0 = r0 + R * (q0 + lq);
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int c = (lbb * NB + q) * 64 + lane;
      const bool okc = j < TBK && c < a.chunks;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t idx = (uint32_t)(n0 + r) * (uint32_t)a.chunks + (uint32_t)c;
        w[q][r] = bload128(rd, okc ? idx * 16u : kNoLoad, 0);
        if constexpr (KIND == K_INT4_24)
          mw[q][r] = bload64(rm, okc ? idx * 8u : kNoLoad, 0);
        else
          mw[q][r] = make_uint2(0, 0);
      }
    }
    if (++lbb == nblk) {
      lbb = 0;
      ++lq;
    }
  };
  uint4 WA[NB][R], WB[NB][R];
  uint2 MA[NB][R], MB_[NB][R];
  load_blk(WA, MA, 0);
  load_blk(WB, MB_, 1);

  // ---- LDS: activations (bf16: as fp16 with the row scale), metadata, selector table ----
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
    if (lane == 0) stab[TABW + wave] = mx;
    __syncthreads();
    uint32_t M16 = 0;
    for (int w = 0; w < wpg; ++w) M16 = max(M16, stab[TABW + w]);
    xfinite = M16 < 0x7F80u;
    const uint32_t emax = M16 >> 7, b = emax > 29u ? emax - 29u : 0u;
    xunscale = __uint_as_float((b + 15u) << 23);
#pragma unroll
    for (int i = 0; i < XR; ++i) xs[i] = xh_convert(xs[i], (b << 7) * 0x00010001u);
  }
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int s = i * nthr + tid;
    if (s < SM) *reinterpret_cast<uint4*>(sb + s * 16) = xs[i];
  }
  if ((uint32_t)(16 * tid) < mbytes) *reinterpret_cast<uint4*>(sb + sa.lds_meta + 16 * tid) = mv;
  if (tid <= rw) *reinterpret_cast<uint32_t*>(sb + sa.lds_rp + 4 * tid) = has_csr ? rpv : 0u;
  if constexpr (LR) {
    const uint32_t kb = (uint32_t)rw * (uint32_t)sa.rank_row_bytes;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t o = 16u * (uint32_t)(tid + i * nthr);
      if (o < kb) *reinterpret_cast<uint4*>(sb + sa.lds_rank + o) = kv[i];
    }
    if (lr4 && (uint32_t)(16 * tid) < (uint32_t)rw * (uint32_t)sa.rsc_row_bytes)
      *reinterpret_cast<uint4*>(sb + sa.lds_rsc + 16 * tid) = ksv;
  }
  if constexpr (KIND == K_INT4_24) {
    if (tid < 16) {
      const uint2 e = seltab_2_4_entry((uint32_t)tid);
      stab[2 * tid] = e.x;
      stab[2 * tid + 1] = e.y;
    }
  }
  __syncthreads();

  // ---- this wavefront's outliers, packed into its LDS region ----
  const int rwa = R * q0, rwb = min(rw, R * (q0 + nqw));  // its rows, relative to r0
  int E0w = 0;
  if (has_csr && nqw > 0) {
    E0w = (int)*reinterpret_cast<const uint32_t*>(sb + sa.lds_rp + 4 * rwa);
    const int E1w = (int)*reinterpret_cast<const uint32_t*>(sb + sa.lds_rp + 4 * rwb);
    const brsrc_t rcol = make_rsrc(a.col, (uint32_t)a.nnz * 4u), rval = make_rsrc(a.val, (uint32_t)a.nnz * 2u);
    uint32_t oc[kStOutLoads], ov[kStOutLoads];
#pragma unroll
    for (int i = 0; i < kStOutLoads; ++i) {
      const int e = E0w + lane + 64 * i;
      const bool ok = e < E1w && lane + 64 * i < sa.out_cap;
      oc[i] = bload32(rcol, ok ? (uint32_t)e * 4u : kNoLoad, 0);
      ov[i] = bload16(rval, ok ? (uint32_t)e * 2u : kNoLoad, 0);
    }
    uint32_t* ob = reinterpret_cast<uint32_t*>(sb + sa.lds_out) + wave * sa.out_cap;
#pragma unroll
    for (int i = 0; i < kStOutLoads; ++i)
      if (lane + 64 * i < sa.out_cap) ob[lane + 64 * i] = (oc[i] & 0xFFFFu) | (ov[i] << 16);
  }

  // ---- per group: tables, multiply, outliers, rank term, reduction ----
  const uint32_t tabbase = (uint32_t)wave * R * RTB;
  auto setup = [&](int q) {  // tables of group q (rows r0 + R (q0 + q) ...)
    if constexpr (LUT) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int rl = R * (q0 + q) + r;  // row relative to r0 (rows past rw read their zero metadata)
        if constexpr (KIND == K_LUT3) {
          const uint4 lv = *reinterpret_cast<const uint4*>(sb + sa.lds_meta + 16 * rl);
          const uint32_t lw[4] = {lv.x, lv.y, lv.z, lv.w};
          const int ca = lane & 7, cb = lane >> 3;
          const uint32_t va = (lw[ca >> 1] >> (16 * (ca & 1))) & 0xFFFFu;
          const uint32_t vb = (lw[cb >> 1] >> (16 * (cb & 1))) & 0xFFFFu;
          stab[(tabbase >> 2) + r * 64 + lane] = va | (vb << 16);
        } else {
          const uint32_t* lw = reinterpret_cast<const uint32_t*>(sb + sa.lds_meta + 32 * rl);
          const uint2 lo = *reinterpret_cast<const uint2*>(lw + 2 * (lane & 3));
          const uint32_t hi = ((lw[(lane >> 2) >> 1] >> (16 * ((lane >> 2) & 1))) & 0xFFFFu) << 16;
          *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(stab) + tabbase + r * RTB + 16 * lane) =
              make_uint4((lo.x & 0xFFFFu) | hi, (lo.x >> 16) | hi, (lo.y & 0xFFFFu) | hi, (lo.y >> 16) | hi);
        }
      }
    }
  };
  // t = x' L_hat: waited for and read once per wavefront, at its first group's end
  float tv[4] = {0.f, 0.f, 0.f, 0.f};
  bool t_read = false;
  const uint32_t target = (LR && a.lr_flag != nullptr) ? lr_target(a.lr_flag, a.lr_epoch) : 0u;
  auto read_t = [&]() {
    if constexpr (LR) {
      const bool t_ok =
          a.lr_flag == nullptr || wait_lowrank(lr_word(a.lr_flag, a.lr_epoch), target, lane, a.lr_max_polls, a.lr_err);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        tv[i] = j < a.rank ? (t_ok ? load_dev(a.t + j) : __builtin_nanf("")) : 0.f;
      }
      if (a.lr_flag != nullptr && a.lr_epoch == 0) {  // recorded launch: this wavefront's reads of t are done
        __builtin_amdgcn_s_waitcnt(0);
        if (lane == 0) lr_reader_done(a.lr_flag, target, sa.row_waves, wg * wpg + wave);
      }
      t_read = true;
    }
  };
  auto x_lds = [&](int k) -> float {
    const int c = k / SPAN, o = k - c * SPAN;
    return act_f32<false>(lds_u16(sdyn, (uint32_t)(c * XS + 2 * o)));  // fp16 (bf16 rows were converted)
  };
  const uint32_t* ob = reinterpret_cast<const uint32_t*>(sb + sa.lds_out) + wave * sa.out_cap;
  auto finalize = [&](int q, const float (&acc)[R]) {
    if constexpr (LR) {
      if (!t_read) read_t();
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int rl = R * (q0 + q) + r, n = r0 + rl;
      float v = acc[r];
      if constexpr (!LUT) v *= (float)__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(sb + sa.lds_meta + 2 * rl));
      if (has_csr && rl < rw) {
        const int e0 = (int)*reinterpret_cast<const uint32_t*>(sb + sa.lds_rp + 4 * rl);
        const int e1 = (int)*reinterpret_cast<const uint32_t*>(sb + sa.lds_rp + 4 * rl + 4);
        for (int e = e0 + lane; e < e1; e += 64) {
          const int ix = e - E0w;
          uint32_t en;
          if (ix < sa.out_cap) en = ob[ix];
          else en = ((uint32_t)a.col[e] & 0xFFFFu) | ((uint32_t)a.val[e] << 16);  // past the staged entries
          v = __builtin_fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(en >> 16)), x_lds((int)(en & 0xFFFFu)), v);
        }
      }
      if constexpr (BF16) v = xfinite ? v * xunscale : __builtin_nanf("");
      if constexpr (LR) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // branch-free: rank indices past the rank read index 0 and add 0
          const int j0 = lane + 64 * i;
          const bool okj = j0 < a.rank;
          const int j = okj ? j0 : 0;
          float rvv;
          if (lr4) {
            const uint32_t byte = sb[sa.lds_rank + rl * sa.rank_row_bytes + (j >> 1)];
            const uint32_t jg = ((uint32_t)j * a.group_mul) >> 16;
            const uint16_t sc = *reinterpret_cast<const uint16_t*>(sb + sa.lds_rsc + rl * sa.rsc_row_bytes + 2 * jg);
            rvv = (float)((int)((byte >> (4 * (j & 1))) & 0xFu) - 8) * (float)__builtin_bit_cast(_Float16, sc);
          } else {
            const uint32_t u = *reinterpret_cast<const uint16_t*>(sb + sa.lds_rank + rl * sa.rank_row_bytes + 2 * j);
            rvv = a.lr_kind == CL_LR_BF16 ? __uint_as_float(u << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)u);
          }
          v = __builtin_fmaf(okj ? tv[i] : 0.f, okj ? rvv : 0.f, v);
        }
      }
      v = wave_sum_dpp(v);
      if (lane == 0 && rl < rw) a.y[n] = v;
    }
  };

  float acc[R] = {0.f, 0.f};
  int cq = 0, cbb = 0;  // group and block being multiplied
  auto comp_blk = [&](const uint4 (&w)[NB][R], const uint2 (&mw)[NB][R], int j) {
    if (j >= TBK) return;
    if (cbb == 0) {
      if (j > 0) {
        finalize(cq - 1, acc);
        acc[0] = acc[1] = 0.f;
      }
      setup(cq);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int p = cbb * NB + q;
      if (p < sa.npass) {
        const int c = p * 64 + lane;
        uint32_t xv[P];
#pragma unroll
        for (int d = 0; d < XD; ++d) {
          const uint4 v = lds_u128(sdyn, (uint32_t)(c * XS + 16 * d));
          xv[4 * d] = v.x;
          xv[4 * d + 1] = v.y;
          xv[4 * d + 2] = v.z;
          xv[4 * d + 3] = v.w;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint32_t wp[P];
          chunk_pairs<KIND, true>(stab, w[q][r], make_uint4(mw[q][r].x, mw[q][r].y, 0, 0), tabbase + (uint32_t)r * RTB,
                                  0u, wp);
#pragma unroll
          for (int jj = 0; jj < P; ++jj) acc[r] = mac2r<false>(wp[jj], xv[jj], acc[r]);
        }
      }
    }
    if (++cbb == nblk) {
      cbb = 0;
      ++cq;
    }
  };
  comp_blk(WA, MA, 0);
  load_blk(WA, MA, 2);
  comp_blk(WB, MB_, 1);
  load_blk(WB, MB_, 3);
  for (int j = 2; j < TBK; j += 2) {
    comp_blk(WA, MA, j);
    load_blk(WA, MA, j + 2);
    comp_blk(WB, MB_, j + 1);
    load_blk(WB, MB_, j + 3);
  }
  if (nqw > 0) finalize(nqw - 1, acc);
  if constexpr (LR) {
    // a recorded launch counts every row wavefront as a reader of t, this one too if it had no group
    if (!t_read && a.lr_flag != nullptr && a.lr_epoch == 0 && lane == 0)
      lr_reader_done(a.lr_flag, target, sa.row_waves, wg * wpg + wave);
  }
}

template <int KIND, bool BF16, int NB, int XR, bool LR>
static void launch_stream_e(const StreamArgs& s, int grid, int threads, int lds, hipStream_t st) {
  if (s.r.clamp || s.r.xscale)
    hipLaunchKernelGGL((decode_stream_kernel<KIND, BF16, NB, XR, LR, true>), dim3(grid), dim3(threads), lds, st, s);
  else
    hipLaunchKernelGGL((decode_stream_kernel<KIND, BF16, NB, XR, LR, false>), dim3(grid), dim3(threads), lds, st, s);
}

template <int KIND, bool BF16, int NB, int XR>
static void launch_stream_l(const StreamArgs& s, int grid, int threads, int lds, hipStream_t st) {
  if (s.r.lr_kind != CL_LR_NONE) launch_stream_e<KIND, BF16, NB, XR, true>(s, grid, threads, lds, st);
  else launch_stream_e<KIND, BF16, NB, XR, false>(s, grid, threads, lds, st);
}

// Slots per thread the staging needs, and the instantiated round sizes.
template <int KIND, bool BF16>
static hipError_t launch_stream_t(const StreamArgs& s, int grid, int threads, int lds, hipStream_t st) {
  const int slots = s.npass * 64 * RowX<KIND>::slots, per = (slots + threads - 1) / threads;
  if (s.npass <= 2) {
    if (per <= 4) launch_stream_l<KIND, BF16, 1, 4>(s, grid, threads, lds, st);
    else if (per <= 8) launch_stream_l<KIND, BF16, 1, 8>(s, grid, threads, lds, st);
    else return hipErrorInvalidConfiguration;
  } else {
    if (per <= 4) launch_stream_l<KIND, BF16, 2, 4>(s, grid, threads, lds, st);
    else if (per <= 8) launch_stream_l<KIND, BF16, 2, 8>(s, grid, threads, lds, st);
    else if (per <= 12) launch_stream_l<KIND, BF16, 2, 12>(s, grid, threads, lds, st);
    else return hipErrorInvalidConfiguration;
  }
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_stream_kind(const StreamArgs& s, int grid, int threads, int lds, bool bf16, hipStream_t st) {
  return bf16 ? launch_stream_t<KIND, true>(s, grid, threads, lds, st) : launch_stream_t<KIND, false>(s, grid, threads, lds, st);
}

// Staging slots per thread at `threads` threads (the host rejects plans above 12).
template <int KIND>
inline int stream_slots_per_thread(int npass, int threads) {
  return (npass * 64 * RowX<KIND>::slots + threads - 1) / threads;
}

}  // namespace cl
