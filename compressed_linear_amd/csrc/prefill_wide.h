// prefill_wide.h -- large-M forward of the 3-bit LUT format on the matrix cores,
// 256-row weight tiles, every wavefront both stages and multiplies.
//
// A workgroup of eight wavefronts owns a tile of 256 weight rows (n) x 128
// activation rows (m) and walks K in steps of 80 (two 40-code chunks).  Per
// step each thread
//   - loads, three steps ahead into a ring of register stages, 2.5 16-byte
//     units of the activation tile, one 16-byte code chunk (one half of the
//     step) of one weight row (a wavefront covers 64 consecutive rows) and at
//     most one outlier entry;
//   - when the step is staged: stores its activation units to LDS, turns its 40
//     codes into 40 values of the MFMA input type with byte permutes over the
//     row's 8 values held in registers (no table lookups), and stores them;
//   - after a barrier in the middle of the step, adds its outlier entry with an
//     LDS packed atomic add;
//   - multiplies: wavefront (wm, wn) owns rows 64 wm.. of m and 64 wn.. of n
//     (2 x 2 blocks of v_mfma_f32_32x32x16), with the operand reads of a half
//     step issued before that half's staging work.
// LDS rows are 176 bytes (11 16-byte units, 10 used): 16 consecutive rows of one
// unit fall in 16 distinct bank groups, so the operand reads are conflict-free.
// Two tile buffers: step t is multiplied from one while step t + 1 is staged in
// the other; two barriers per step.
//
// Outliers ("SqueezeLLM: Dense-and-Sparse Quantization", Approach: W = D + S)
// come as per-(256-row tile, step) lists built when the layer is created
// (entry: row | k in step << 8 | fp16 value << 16).  The rank-r correction
// ("SLiM" page, review highlights: y += (x' L) R) runs as extra K steps over
// [t_hi | t_lo] x [R^T | R^T], t = x' L computed beforehand.
//
// Compared with the 128 x 128 kernel with separate staging wavefronts, every
// weight is dequantised once per 128 activation rows as before, but the 256-row
// weight tile halves the activation traffic per weight, the dequantisation uses
// no LDS lookups, and all eight wavefronts issue MFMAs.
#pragma once
#include <hip/hip_runtime.h>

#include "prefill_impl.h"

namespace cl {

constexpr int kPwBN = 256, kPwBM = 128, kPwBK = 80;  // weight rows, activation rows, K per step
constexpr int kPwRS = 176;                           // LDS bytes per tile row (11 units)
constexpr int kPwTA = kPwBM * kPwRS, kPwTB = kPwBN * kPwRS, kPwStage = kPwTA + kPwTB;
constexpr int kPwBuf = ((kPfMaxSteps + 1) * 4 + 15) / 16 * 16;  // tile buffers after the outlier offsets
constexpr int kPwLds = kPwBuf + 2 * kPwStage;
constexpr int kPwAU = 3;                             // activation units per thread per step (1280 units)
static_assert(kPwLds <= 160 * 1024, "LDS budget");

// One outlier entry (row | k << 8 | fp16 value << 16) into the weight tile at
// byte offset btile, packed atomic add on the dword holding it.
template <bool BF16>
__device__ __forceinline__ void pw_add_outlier(uint8_t* smem, uint32_t btile, uint32_t e) {
  const uint32_t row = e & 255u, kl = (e >> 8) & 127u;
  const uint32_t addr = btile + row * kPwRS + (kl & ~1u) * 2u;
  const uint32_t v16 = to16<BF16>((float)__builtin_bit_cast(_Float16, (uint16_t)(e >> 16)));
  const uint32_t pk = (kl & 1u) ? (v16 << 16) : v16;
  void* q = smem + addr;
  if constexpr (BF16)
    __builtin_amdgcn_ds_atomic_fadd_v2bf16((__attribute__((address_space(3))) pf_bf16x2*)q,
                                           __builtin_bit_cast(pf_bf16x2, pk));
  else
    __builtin_amdgcn_ds_atomic_fadd_v2f16((__attribute__((address_space(3))) pf_f16x2*)q,
                                          __builtin_bit_cast(pf_f16x2, pk));
}

template <bool BF16>
__global__ void __launch_bounds__(512, 1) prefill_wide_kernel(PfArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kPwLds];
  int32_t* s_cptr = reinterpret_cast<int32_t*>(smem);
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Tile order: the blocks one XCD receives (blockIdx mod 8) take consecutive
  // ids, and consecutive ids cover groups of 8 weight tiles x every activation
  // tile, so the workgroups running together on an XCD share activation and
  // code lines in its L2.
  const int tiles_n = (a.ncols + kPwBN - 1) / kPwBN, tiles_m = (a.M + kPwBM - 1) / kPwBM;
  const int nb = tiles_n * tiles_m, b = (int)blockIdx.x;
  const int v = (nb & 7) == 0 ? (b & 7) * (nb >> 3) + (b >> 3) : b;
  const int GN = (tiles_n & 7) == 0 ? 8 : 1;
  const int grp = v / (GN * tiles_m), rem = v - grp * (GN * tiles_m);
  const int tm = rem / GN, tn = grp * GN + (rem - (rem / GN) * GN);
  const int n0 = tn * kPwBN, m0 = tm * kPwBM;
  const bool has_csr = a.cptr != nullptr;
  const int nd = a.nsteps_dense;

  if (has_csr) {
    const int32_t* cp = a.cptr + (size_t)tn * (nd + 1);
    for (int i = tid; i <= nd; i += 512) s_cptr[i] = cp[i];
  }
  // this thread's weight row and chunk half (a wavefront stages 64 consecutive
  // rows of one half, so its 16-byte LDS stores hit distinct bank groups), and
  // the row's values as byte tables
  const int srow = (tid & 63) + 64 * (tid >> 7), shalf = (tid >> 6) & 1, n = n0 + srow;
  const Lut3Bytes T =
      lut3_bytes<BF16>(n < a.Npad ? reinterpret_cast<const uint4*>(a.table)[n] : make_uint4(0, 0, 0, 0));
  __syncthreads();

  const brsrc_t rx = make_rsrc(a.x, (uint32_t)a.M * (uint32_t)a.ldx * 2u);
  const brsrc_t rd = make_rsrc(a.dense, (uint32_t)a.Npad * (uint32_t)a.chunks * 16u);
  // (the size read back from LDS is uniform; readfirstlane keeps the descriptor
  // in scalar registers, without a waterfall loop around every load through it)
  const brsrc_t rc = make_rsrc(a.cent, has_csr ? (uint32_t)__builtin_amdgcn_readfirstlane(s_cptr[nd]) * 4u : 0u);
  const uint32_t wrow = (uint32_t)n * (uint32_t)a.chunks;
  // activation units of this thread (u = tid + 512 i of the 128 x 10 units of a
  // step): element offset of the unit at step 0, k in step, LDS byte offset.
  // Threads past the 1280 units store zeros into the unused 11th unit of a
  // weight-tile row instead, so the staging has no branch.
  // xend: the unit is loaded at steps s < xend (inside the dense steps and below ldx)
  uint32_t xoff[kPwAU], xlds[kPwAU];
  int xend[kPwAU];
#pragma unroll
  for (int i = 0; i < kPwAU; ++i) {
    const int u = tid + 512 * i;
    const bool in = u < kPwBM * 10;
    const int row = in ? u / 10 : 0, kk = in ? u - row * 10 : 0;
    const int e = (a.ldx - 8 * kk + kPwBK - 1) / kPwBK;
    xend[i] = in ? (e < nd ? e : nd) : 0;
    xoff[i] = ((uint32_t)(m0 + row) * (uint32_t)a.ldx + (uint32_t)(8 * kk)) * 2u;
    xlds[i] = in ? (uint32_t)(row * kPwRS + kk * 16) : (uint32_t)(kPwTA + (u - kPwBM * 10) * kPwRS + 160);
  }
  // the code chunk 2 s + shalf exists for steps s < cend
  const int cend = (a.chunks - shalf + 1) / 2 < nd ? (a.chunks - shalf + 1) / 2 : nd;

  struct Stage {
    uint4 xa[kPwAU];
    uint4 wb;
    uint32_t ce;
    bool ce_ok;
  };
  // Every load of a step is issued whatever the step: invalid ones read through a
  // poisoned offset (outside the buffer, zero), so the compiler waits for exactly
  // the stage it consumes while the younger stages stay in flight.
  auto load_step = [&](Stage& st, int s, bool valid) {
#pragma unroll
    for (int i = 0; i < kPwAU; ++i)
      st.xa[i] = bload128(rx, s < xend[i] ? xoff[i] + (uint32_t)(s * kPwBK * 2) : kNoLoad, 0);
    st.wb = bload128(rd, s < cend ? (wrow + (uint32_t)(2 * s + shalf)) * 16u : kNoLoad, 0);
    const int sc = valid ? s : 0;
    const int e0 = has_csr ? s_cptr[sc] : 0, cnt = has_csr ? s_cptr[sc + 1] - e0 : 0;
    st.ce_ok = has_csr && valid && tid < cnt;
    st.ce = bload32(rc, st.ce_ok ? (uint32_t)(e0 + tid) * 4u : kNoLoad, 0);
  };
  auto stage_dense = [&](const Stage& st, int buf) {
    uint8_t* bo = smem + kPwBuf + buf * kPwStage;
#pragma unroll
    for (int i = 0; i < kPwAU; ++i) *reinterpret_cast<uint4*>(bo + xlds[i]) = st.xa[i];
    uint32_t wp[20];
    const uint32_t ww[4] = {st.wb.x, st.wb.y, st.wb.z, st.wb.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) lut3_word_perm(ww[i], T, &wp[5 * i]);
    uint8_t* brow = bo + kPwTA + srow * kPwRS + shalf * 80;
#pragma unroll
    for (int j = 0; j < 5; ++j)
      *reinterpret_cast<uint4*>(brow + 16 * j) = make_uint4(wp[4 * j], wp[4 * j + 1], wp[4 * j + 2], wp[4 * j + 3]);
  };
  // rank step s: activations t_hi | t_lo and weights R^T | R^T, loaded directly
  auto stage_rank = [&](int s, int buf) {
    uint8_t* bo = smem + kPwBuf + buf * kPwStage;
    const int k0 = (s - nd) * kPwBK;
    const brsrc_t ra = make_rsrc(a.a2, (uint32_t)a.M * (uint32_t)a.lda2 * 2u);
    const brsrc_t rr = make_rsrc(a.r16, (uint32_t)a.Npad * (uint32_t)a.ldr16 * 2u);
    uint4 va[kPwAU], vb[5];
#pragma unroll
    for (int i = 0; i < kPwAU; ++i) {
      const int u = tid + 512 * i, row = u / 10, kk = u - row * 10, k = k0 + 8 * kk;
      const bool ok = u < kPwBM * 10 && k < a.lda2;
      va[i] = bload128(ra, ok ? ((uint32_t)(m0 + row) * (uint32_t)a.lda2 + (uint32_t)k) * 2u : kNoLoad, 0);
    }
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int k = k0 + shalf * 40 + 8 * j;
      vb[j] = bload128(rr, k < a.ldr16 ? ((uint32_t)n * (uint32_t)a.ldr16 + (uint32_t)k) * 2u : kNoLoad, 0);
    }
#pragma unroll
    for (int i = 0; i < kPwAU; ++i) {
      const int u = tid + 512 * i, row = u / 10, kk = u - row * 10;
      if (u < kPwBM * 10) *reinterpret_cast<uint4*>(bo + row * kPwRS + kk * 16) = va[i];
    }
    uint8_t* brow = bo + kPwTA + srow * kPwRS + shalf * 80;
#pragma unroll
    for (int j = 0; j < 5; ++j) *reinterpret_cast<uint4*>(brow + 16 * j) = vb[j];
  };
  auto add_outlier1 = [&](const Stage& st, int buf) {
    if (has_csr && st.ce_ok) pw_add_outlier<BF16>(smem, (uint32_t)(kPwBuf + buf * kPwStage + kPwTA), st.ce);
  };
  auto add_outliers_rest = [&](int s, int buf) {  // lists longer than one entry per thread
    if (!has_csr) return;
    const int e0 = s_cptr[s], cnt = s_cptr[s + 1] - e0;
    for (int i = 512 + tid; i < cnt; i += 512)
      pw_add_outlier<BF16>(smem, (uint32_t)(kPwBuf + buf * kPwStage + kPwTA), a.cent[e0 + i]);
  };
  auto add_outliers = [&](const Stage& st, int s, int buf) {
    if (s >= nd) return;
    add_outlier1(st, buf);
    add_outliers_rest(s, buf);
  };


  // ---- multiply: wavefront (wm, wn) owns 64 x 64 of the 128 x 256 tile ----
  const int wm = wave >> 2, wn = wave & 3;
  pf_f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const uint32_t ar = (uint32_t)((wm * 64 + (lane & 31)) * kPwRS + (lane >> 5) * 16);
  const uint32_t br = (uint32_t)(kPwTA + (wn * 64 + (lane & 31)) * kPwRS + (lane >> 5) * 16);
  auto mma = [&](int buf, int ks0, int ks1) {
    const uint8_t* bo = smem + kPwBuf + buf * kPwStage;
    uint4 fa[2][2], fb[2][2];
    auto rd = [&](int ks, int q) {
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[q][i] = *reinterpret_cast<const uint4*>(bo + ar + i * 32 * kPwRS + ks * 32);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[q][j] = *reinterpret_cast<const uint4*>(bo + br + j * 32 * kPwRS + ks * 32);
    };
    rd(ks0, 0);
#pragma unroll
    for (int ks = ks0; ks < ks1; ++ks) {
      const int q = (ks - ks0) & 1;
      if (ks + 1 < ks1) rd(ks + 1, q ^ 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = pf_mfma<BF16>(fa[q][i], fb[q][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- the step loop: ring of three register stages, step t+1 staged while t is
  // multiplied.  Dense steps run a loop of their own with no branch on the step's
  // kind, so the compiler's waits stay exact (the ring's younger stages in flight);
  // the rank steps follow with direct loads.
  const int ns = a.nsteps;
  Stage S0, S1, S2;
  load_step(S0, 0, 0 < nd);
  load_step(S1, 1, 1 < nd);
  load_step(S2, 2, 2 < nd);
  stage_dense(S0, 0);
  __syncthreads();
  add_outliers(S0, 0, 0);
  load_step(S0, 3, 3 < nd);
  // Dense iteration: the operand reads of a half step are issued before the
  // staging stores, so that the dequantisation's vector instructions and the
  // MFMAs carry no memory dependence on each other and the compiler can
  // interleave them.  (A forced pattern of one MFMA then eight vector
  // instructions measured 1-2 % slower; an outlier add issued by every thread,
  // zero for threads without an entry, to drop the branch: 22 % slower.)
  auto iter_dense = [&](Stage& nx, int t) {  // t + 1 < nd
    __syncthreads();  // step t's tile and outliers are in place; step t-1's reads are done
    const uint8_t* cb = smem + kPwBuf + (t & 1) * kPwStage;
    uint4 f[3][4];
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      f[ks][0] = *reinterpret_cast<const uint4*>(cb + ar + ks * 32);
      f[ks][1] = *reinterpret_cast<const uint4*>(cb + ar + 32 * kPwRS + ks * 32);
      f[ks][2] = *reinterpret_cast<const uint4*>(cb + br + ks * 32);
      f[ks][3] = *reinterpret_cast<const uint4*>(cb + br + 32 * kPwRS + ks * 32);
    }
    stage_dense(nx, (t + 1) & 1);
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      acc[0][0] = pf_mfma<BF16>(f[ks][0], f[ks][2], acc[0][0]);
      acc[0][1] = pf_mfma<BF16>(f[ks][0], f[ks][3], acc[0][1]);
      acc[1][0] = pf_mfma<BF16>(f[ks][1], f[ks][2], acc[1][0]);
      acc[1][1] = pf_mfma<BF16>(f[ks][1], f[ks][3], acc[1][1]);
    }
    __syncthreads();  // step t+1's tile has landed
    uint4 g[2][4];
#pragma unroll
    for (int ks = 3; ks < 5; ++ks) {
      g[ks - 3][0] = *reinterpret_cast<const uint4*>(cb + ar + ks * 32);
      g[ks - 3][1] = *reinterpret_cast<const uint4*>(cb + ar + 32 * kPwRS + ks * 32);
      g[ks - 3][2] = *reinterpret_cast<const uint4*>(cb + br + ks * 32);
      g[ks - 3][3] = *reinterpret_cast<const uint4*>(cb + br + 32 * kPwRS + ks * 32);
    }
    add_outlier1(nx, (t + 1) & 1);
    load_step(nx, t + 4, t + 4 < nd);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      acc[0][0] = pf_mfma<BF16>(g[ks][0], g[ks][2], acc[0][0]);
      acc[0][1] = pf_mfma<BF16>(g[ks][0], g[ks][3], acc[0][1]);
      acc[1][0] = pf_mfma<BF16>(g[ks][1], g[ks][2], acc[1][0]);
      acc[1][1] = pf_mfma<BF16>(g[ks][1], g[ks][3], acc[1][1]);
    }
    add_outliers_rest(t + 1, (t + 1) & 1);
  };
  auto iter_rank = [&](int t) {  // t + 1 >= nd
    __syncthreads();
    if (t + 1 < ns) stage_rank(t + 1, (t + 1) & 1);
    mma(t & 1, 0, 3);
    __syncthreads();
    mma(t & 1, 3, 5);
  };
  int t = 0;
  for (; t + 3 < nd; t += 3) {
    iter_dense(S1, t);
    iter_dense(S2, t + 1);
    iter_dense(S0, t + 2);
  }
  if (t + 1 < nd) {
    iter_dense(S1, t++);
    if (t + 1 < nd) iter_dense(S2, t++);
  }
  for (; t < ns; ++t) iter_rank(t);

  // ---- store: lane l of block (i, j) holds column n = l mod 32, rows 8 (v/4) + 4 (l/32) + v mod 4 ----
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int nn = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m < a.M && nn < a.ncols) a.y[(size_t)m * a.ldy + nn] = acc[i][j][e];
      }
    }
}

}  // namespace cl
