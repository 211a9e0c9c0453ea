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
// every load a wavefront needs is issued before it waits for any of them
// (row pointers and LUT values first, then the code stream in blocks of NB
// passes, two blocks in flight), and nothing that depends on a load sits in
// front of the code stream.  The activations are staged once per workgroup in
// LDS (chunk c of row m at c * XS bytes, XS the chunk's activation bytes padded
// so that eight lanes' 16-byte reads fall in distinct banks), which keeps them
// out of the registers and lets the outlier gather read LDS instead of memory.
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
  int npass;  // ceil(chunks / 64)
  int xrow;   // LDS bytes per staged activation row (npass * 64 chunks)
  int lds_t;  // byte offset of the low-rank intermediate in LDS
  int lds_x;  // byte offset of the staged activations in LDS
};

// LDS bytes per chunk of staged activations: 2 * span rounded up to 16 * (odd
// multiple of 1 in dwords mod 8), so lanes 0..7 of a 128-bit read hit 8
// distinct groups of four banks.
template <int KIND>
struct RowX {
  static constexpr int span = KindTraits<KIND>::span;
  static constexpr int stride = span == 40 ? 80 : span == 32 ? 80 : span == 64 ? 144 : 48;
  static constexpr int slots = stride / 16;  // 16-byte slots per chunk
};

// LDS bytes of the row tables in front of t: per wavefront R regions of 256 bytes
// (LUT formats), the shared 2:4 selector table, or nothing.
template <int KIND, int R>
constexpr int row_tab_bytes() {
  return (KIND == K_LUT3 || KIND == K_LUT4) ? 4 * R * 256 : KIND == K_INT4_24 ? 256 : 0;
}

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

__device__ __forceinline__ uint4 lds_u128(const uint32_t* lds, uint32_t byte_addr) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(lds) + byte_addr);
}

// R = rows per wavefront, MB = activation rows (M <= MB), NB = passes per block.
template <int KIND, int MB, bool BF16, int R, int NB>
__global__ void __launch_bounds__(256) decode_rows_kernel(RowArgs a) {
  constexpr int SPAN = KindTraits<KIND>::span, P = KindTraits<KIND>::pairs, XD = SPAN / 8;  // 16-byte x slots per chunk
  constexpr int XS = RowX<KIND>::stride, XSL = RowX<KIND>::slots;
  constexpr bool LUT = KIND == K_LUT3 || KIND == K_LUT4;
  extern __shared__ uint32_t smem[];  // the only LDS object: starts at address 0
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int row0 = (blockIdx.x * 4 + wave) * R;  // < Npad (the grid covers Npad exactly)
  const uint32_t tabbase = (uint32_t)(wave * R * 256);
  const bool has_csr = a.rowptr != nullptr, has_lr = a.lr_kind != CL_LR_NONE;

  // ---- scalar loads: row pointers (uniform) ----
  int e0[R], e1[R];
  {
    typedef const __attribute__((address_space(4))) int32_t* sp;
    const sp rp = (sp)a.rowptr;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      e0[r] = has_csr ? rp[min(row0 + r, a.N)] : 0;
      e1[r] = has_csr ? rp[min(row0 + r + 1, a.N)] : 0;
    }
  }
  // ---- LUT values (or the integer row scales) ----
  uint32_t tv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if constexpr (KIND == K_LUT4) {
      tv[r] = a.table[(size_t)(row0 + r) * 16 + (lane & 15)];
    } else if constexpr (KIND == K_LUT3) {
      const uint16_t* lt = a.table + (size_t)(row0 + r) * 8;
      tv[r] = (uint32_t)lt[lane & 7] | ((uint32_t)lt[lane >> 3] << 16);  // pair entry (a, b) = lane
    } else {
      tv[r] = a.table[row0 + r];  // fp16 row scale
    }
  }

  // ---- activations, first round: issued before the code stream so that
  // waiting for them does not wait for the codes ----
  constexpr int XR0 = 8;  // 16-byte slots per thread in the first round
  const int xch = a.npass * 64;  // staged chunks per row
  const int xslots = MB * xch * XSL;
  const uint16_t* xg = static_cast<const uint16_t*>(a.x);
  auto x_slot = [&](int s) -> uint4 {
    const int m = s / (xch * XSL), rem = s - m * (xch * XSL), c = rem / XSL, d = rem - c * XSL;
    const int k = c * SPAN + 8 * d;
    const bool ok = s < xslots && d < XD && m < a.M && k < a.ldx;  // ldx: a multiple of 8, zero past K
    return ok ? *reinterpret_cast<const uint4*>(xg + (size_t)m * a.ldx + k) : make_uint4(0, 0, 0, 0);
  };
  auto x_store = [&](int s, uint4 v) {
    if (s < xslots) {
      const int m = s / (xch * XSL), rem = s - m * (xch * XSL);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(smem) + a.lds_x + m * a.xrow + rem * 16) = v;
    }
  };
  uint4 xs0[XR0];
#pragma unroll
  for (int i = 0; i < XR0; ++i) xs0[i] = x_slot(i * 256 + tid);

  // ---- the code stream: two blocks of NB passes in flight ----
  const int nblk = (a.npass + NB - 1) / NB;
  auto load_blk = [&](uint4 (&w)[NB][R], uint2 (&mw)[NB][R], int b) {
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int c = (b * NB + q) * 64 + lane;
      const bool ok = b < nblk && c < a.chunks;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const size_t idx = (size_t)(row0 + r) * a.chunks + c;
        w[q][r] = ok ? a.dense[idx] : make_uint4(0, 0, 0, 0);
        if constexpr (KIND == K_INT4_24)
          mw[q][r] = ok ? reinterpret_cast<const uint2*>(a.meta)[idx] : make_uint2(0, 0);
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
  int ccol[R];
  float cval[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = e0[r] + lane;
    const bool ok = e < e1[r];
    ccol[r] = ok ? a.col[e] : 0;
    cval[r] = ok ? (float)__builtin_bit_cast(_Float16, a.val[e]) : 0.f;
  }
  float rv[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = lane + 64 * i, n = row0 + r;
      float v = 0.f;
      if (has_lr && j < a.rank) {
        if (a.lr_kind == CL_LR_INT4) {  // R^T codes [Npad][ceil(r/2)], scales [Npad][ceil(r/g)]
          const int gr = (a.rank + a.group - 1) / a.group;
          const uint32_t byte = a.R[(size_t)n * ((a.rank + 1) >> 1) + (j >> 1)];
          const int qv = (int)((byte >> (4 * (j & 1))) & 0xFu) - 8;
          v = (float)qv * (float)__builtin_bit_cast(_Float16, a.Rscale[(size_t)n * gr + j / a.group]);
        } else {  // R^T [Npad][r]
          const uint16_t u = reinterpret_cast<const uint16_t*>(a.R)[(size_t)n * a.rank + j];
          v = a.lr_kind == CL_LR_BF16 ? __uint_as_float((uint32_t)u << 16) : (float)__builtin_bit_cast(_Float16, u);
        }
      }
      rv[r][i] = v;
    }

  // ---- stage the activations (and t) in LDS, zero past K and past M ----
  {
#pragma unroll
    for (int i = 0; i < XR0; ++i) x_store(i * 256 + tid, xs0[i]);
    for (int s0 = XR0 * 256; s0 < xslots; s0 += 4 * 256) {
      uint4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = x_slot(s0 + i * 256 + tid);
#pragma unroll
      for (int i = 0; i < 4; ++i) x_store(s0 + i * 256 + tid, v[i]);
    }
    if (has_lr) {
      float* s_t = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(smem) + a.lds_t);
      for (int i = tid; i < MB * 256; i += 256) {
        const int m = i >> 8, j = i & 255;
        s_t[i] = (j < a.rank && m < a.M) ? a.t[m * a.rank + j] : 0.f;
      }
    }
  }
  // ---- tables: per-wavefront row tables, or the shared selector table ----
  if constexpr (KIND == K_LUT4) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (lane < 16) smem[(tabbase >> 2) + r * 64 + lane] = tv[r];
  } else if constexpr (KIND == K_LUT3) {
#pragma unroll
    for (int r = 0; r < R; ++r) smem[(tabbase >> 2) + r * 64 + lane] = tv[r];
  } else if constexpr (KIND == K_INT4_24) {
    if (tid < 16) {
      const uint2 e = seltab_2_4_entry((uint32_t)tid);
      smem[2 * tid] = e.x;
      smem[2 * tid + 1] = e.y;
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
            const uint4 v = lds_u128(smem, (uint32_t)(a.lds_x + m * a.xrow + c * XS + 16 * d));
            xv[m][4 * d] = v.x;
            xv[m][4 * d + 1] = v.y;
            xv[m][4 * d + 2] = v.z;
            xv[m][4 * d + 3] = v.w;
          }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint32_t wp[P];
          chunk_pairs<KIND, true>(smem, w[q][r], make_uint4(mw[q][r].x, mw[q][r].y, 0, 0), tabbase + (uint32_t)(r * 256),
                                  0u, wp);
#pragma unroll
          for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int j = 0; j < P; ++j) acc[r][m] = mac2r<BF16>(wp[j], xv[m][j], acc[r][m]);
        }
      }
    }
  };
  for (int b = 0; b < nblk; b += 2) {
    comp_blk(WA, MA, b);
    if (b + 2 < nblk) load_blk(WA, MA, b + 2);
    if (b + 1 < nblk) {
      comp_blk(WB, MB_, b + 1);
      if (b + 3 < nblk) load_blk(WB, MB_, b + 3);
    }
  }

  // ---- integer formats: the row scale multiplies the dense part only ----
  if constexpr (!LUT) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)tv[r]);
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[r][m] *= sc;
    }
  }
  // ---- outliers: activations gathered from LDS ----
  auto x_lds = [&](int m, int k) -> float {
    const int c = k / SPAN, o = k - c * SPAN;
    return act_f32<BF16>(lds_u16(smem, (uint32_t)(a.lds_x + m * a.xrow + c * XS + 2 * o)));
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
  // ---- rank terms: t (LDS) times R^T ----
  if (has_lr) {
    const float* s_t = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(smem) + a.lds_t);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[r][m] = __builtin_fmaf(s_t[m * 256 + lane + 64 * i], rv[r][i], acc[r][m]);
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

// Largest LDS a row-wise workgroup may take; larger activation blocks go to the tile kernel.
constexpr int kRowsMaxLds = 64 * 1024;

template <int KIND, int MB, int R>
inline int rows_lds_layout(RowArgs& a) {
  a.npass = (a.chunks + 63) / 64;
  a.xrow = a.npass * 64 * RowX<KIND>::stride;
  a.lds_t = row_tab_bytes<KIND, R>();
  a.lds_x = a.lds_t + (a.lr_kind != CL_LR_NONE ? MB * 256 * 4 : 0);
  return a.lds_x + MB * a.xrow;
}

template <int KIND, int MB, bool BF16, int R>
static hipError_t launch_rows_t(RowArgs a, int Npad, hipStream_t st) {
  const int lds = rows_lds_layout<KIND, MB, R>(a);
  if (lds > kRowsMaxLds) return hipErrorInvalidConfiguration;
  const int grid = Npad / (4 * R);  // Npad is a multiple of 64, so of 4 * R
  hipLaunchKernelGGL((decode_rows_kernel<KIND, MB, BF16, R, 2>), dim3(grid), dim3(256), lds, st, a);
  return hipGetLastError();
}

// Whether the row-wise kernel takes this shape (its staged activations fit in LDS).
template <int KIND>
bool rows_fit(RowArgs a) {
  const int mb = a.M <= 1 ? 1 : a.M <= 2 ? 2 : 4;
  const int lds = mb == 1 ? rows_lds_layout<KIND, 1, 2>(a) : mb == 2 ? rows_lds_layout<KIND, 2, 1>(a)
                                                                     : rows_lds_layout<KIND, 4, 1>(a);
  return lds <= kRowsMaxLds;
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
