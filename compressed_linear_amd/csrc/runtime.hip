// runtime.hip -- the C ABI: upload, forward dispatch, debug dequantisation.
#include <hip/hip_runtime.h>

#include <cstring>
#include <new>
#include <vector>

#include "internal.h"
#include "layer.h"

namespace cl {

// Split-K workgroups per tile of the tile kernel: enough workgroups for about
// two per CU, each wave still streaming at least a few chunks.
static int choose_split(const cl_blob_header& h, int num_cus) {
  const int target = 2 * num_cus;
  int s = (int)((target + h.n_tiles / 2) / h.n_tiles);
  const int max_by_chunks = h.chunks / (4 * 2) > 0 ? h.chunks / (4 * 2) : 1;
  if (s > max_by_chunks) s = max_by_chunks;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return s;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Which decode low-rank prologue a layer takes: 0 for 16-bit L of the
// activation type (pairwise dot products), 1 for int4 L with groups of at
// least 16 along K (at most 33 scale rows per K slice), else -1 (per-column kernel).
static int lowrank_mode(const cl_blob_header& h) {
  if (h.lr == CL_LR_NONE || h.rank <= 0) return -1;
  if (h.lr == CL_LR_INT4) return h.group >= 16 ? 1 : -1;
  const bool lbf = h.lr == CL_LR_BF16, xbf = h.x_dtype == CL_ACT_BF16;
  return lbf == xbf ? 0 : -1;
}

size_t workspace_layout(const cl_blob_header& h, int32_t max_M, Layer* L, size_t base, size_t* largest) {
  const int split = L ? L->split : 64;  // size query: the largest split
  const int Npad = h.n_tiles * 64;
  size_t off = align256(base), big = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    if (bytes > big) big = bytes;
    return o;
  };
  const int mblocks = (int)ceil_div(max_M, 32);
  const size_t o_cnt = take((size_t)(h.n_tiles + mblocks + 8) * 4);
  const size_t o_part = take((size_t)h.n_tiles * split * kMaxDecodeM * 64 * 4);
  size_t o_nzs = 0, o_t = 0, o_xp = 0;
  if (h.mask == CL_MASK_BITMAP) o_nzs = take((size_t)Npad * 4 * split * 4);
  // t = x' L: [max_M][rank] for decode; prefill keeps up to 8 K-split partials [8][max_M][rank rounded to 8]
  if (h.lr != CL_LR_NONE && h.rank > 0) o_t = take((size_t)8 * max_M * round_up(h.rank, 8) * 4);
  // activations are restaged (clamped and / or channel-scaled, row stride a
  // multiple of 8 for aligned 128-bit loads) when the layer clamps or scales
  // them or K is not a multiple of 8
  const int Kx = (int)round_up(h.K, 8);
  if (h.has_clamp || h.n_xscale > 0 || (h.K & 7)) o_xp = take((size_t)max_M * Kx * 2);
  // matrix-core prefill: outlier lists per (128-row tile, K step), R^T twice
  // and L^T in the MFMA input type, t_hi | t_lo.  A bitmap layer created for
  // batches above the decode range runs the INT8 tile loader on a dense int8
  // copy of its weights (zero where dropped); otherwise it keeps only R^T twice
  // (its decode runs on the matrix-core kernel)
  size_t o_pfp = 0, o_pfe = 0, o_pfr = 0, o_pfl = 0, o_pft = 0, o_pfd = 0;
  int pf_nd = 0, pf_chunks8 = 0;
  const int rp = (int)round_up(h.rank, 8);
  const bool has_lr = h.lr != CL_LR_NONE && h.rank > 0;
  const bool bm_prefill = h.mask == CL_MASK_BITMAP && max_M > kMaxDecodeM;
  if (h.mask != CL_MASK_BITMAP || bm_prefill) {
    const int pmask = bm_prefill ? CL_MASK_NONE : h.mask;
    const int span = kind_info(h.dense, pmask).span;
    const int chunks = bm_prefill ? (int)ceil_div(h.K, span) : h.chunks;
    const int cps = pf_step_k(h.dense, pmask) / span;
    pf_nd = (int)ceil_div(chunks, cps);
    if (bm_prefill) {
      pf_chunks8 = chunks;
      o_pfd = take((size_t)Npad * chunks * 16);
    }
    if (h.nnz > 0) {
      o_pfp = take((size_t)ceil_div(Npad, pf_tile_rows(h.dense)) * (pf_nd + 1) * 4);
      o_pfe = take((size_t)h.nnz * 4);
    }
    if (has_lr) {
      o_pfr = take((size_t)Npad * 2 * rp * 2);
      o_pfl = take((size_t)h.rank * Kx * 2);
      o_pft = take((size_t)max_M * 2 * rp * 2);
    }
  } else if (has_lr) {
    o_pfr = take((size_t)Npad * 2 * rp * 2);
  }
  // matrix-core decode: slice partial sums, outlier lists per (slice, tile, row)
  size_t o_mfp = 0, o_mfo = 0, o_mfe = 0, o_mfz = 0;
  int mf_npw = 0, mf_Kz = 0, mf_S = 0, mf_tiles = 0;
  // (bitmap layers at any max_M: the kernel is their decode path at every batch)
  if (max_M >= 2 || h.mask == CL_MASK_BITMAP) {
    mf_npw = mf_passes(h.dense, h.mask, h.K, h.N);
    mf_Kz = mf_npw * mf_pass_k(h.dense, h.mask);
    mf_tiles = (int)ceil_div(h.N, kMfRows);
    mf_S = (int)ceil_div(h.K, mf_Kz);
    o_mfp = take((size_t)mf_tiles * mf_S * 32 * kMfRows * 4);
    if (h.nnz > 0) {
      o_mfo = take(((size_t)mf_S * mf_tiles * kMfRows + 1) * 4);
      o_mfe = take((size_t)h.nnz * 4);
    }
    if (h.mask == CL_MASK_BITMAP) o_mfz = take((size_t)Npad * mf_S * 4);
  }
  // decode low-rank prologue: k-major copy of L, partial sums, arrival counters
  size_t o_lk = 0, o_ls = 0, o_lp = 0, o_lc = 0, lp_bytes = 0;
  const int lr_mode = lowrank_mode(h);
  const int lr_rpad = (int)round_up(h.rank > 0 ? h.rank : 1, 64), lr_S = (int)ceil_div(h.K, kLrSlice);
  if (has_lr && lr_mode >= 0) {
    const size_t Kl = (size_t)lr_S * kLrSlice;
    o_lk = take(lr_mode == 0 ? Kl * lr_rpad * 2 : Kl / 2 * lr_rpad);
    if (lr_mode == 1) o_ls = take((size_t)ceil_div(Kl, h.group) * lr_rpad * 2);
    const int mt = (int)ceil_div(max_M < kMaxDecodeM ? max_M : kMaxDecodeM, 4);
    lp_bytes = (size_t)(lr_rpad / 64) * mt * lr_S * 256 * 4;
    o_lp = take(lp_bytes);
    o_lc = take(kLrCntWords * 4);
  }
  if (L) {
    uint8_t* d = L->dev;
    L->lr_mode = (has_lr && lr_mode >= 0) ? lr_mode : -1;
    L->lr_rpad = lr_rpad;
    L->lr_S = lr_S;
    L->lr_lk = o_lk ? d + o_lk : nullptr;
    L->lr_ls = o_ls ? reinterpret_cast<uint16_t*>(d + o_ls) : nullptr;
    L->lr_part = o_lp ? reinterpret_cast<float*>(d + o_lp) : nullptr;
    L->lr_part_bytes = lp_bytes;
    L->lr_cnt = o_lc ? reinterpret_cast<uint32_t*>(d + o_lc) : nullptr;
    L->counters = reinterpret_cast<uint32_t*>(d + o_cnt);
    L->part = reinterpret_cast<float*>(d + o_part);
    L->nzstart = o_nzs ? reinterpret_cast<int32_t*>(d + o_nzs) : nullptr;
    L->t = o_t ? reinterpret_cast<float*>(d + o_t) : nullptr;
    L->xprep = o_xp ? reinterpret_cast<uint16_t*>(d + o_xp) : nullptr;
    L->Kx = Kx;
    L->pf_nd = pf_nd;
    L->pf_dense8 = o_pfd ? d + o_pfd : nullptr;
    L->pf_chunks8 = pf_chunks8;
    L->pf_cptr = o_pfp ? reinterpret_cast<int32_t*>(d + o_pfp) : nullptr;
    L->pf_cent = o_pfe ? reinterpret_cast<uint32_t*>(d + o_pfe) : nullptr;
    L->pf_r16 = o_pfr ? reinterpret_cast<uint16_t*>(d + o_pfr) : nullptr;
    L->pf_l16 = o_pfl ? reinterpret_cast<uint16_t*>(d + o_pfl) : nullptr;
    L->pf_t16 = o_pft ? reinterpret_cast<uint16_t*>(d + o_pft) : nullptr;
    L->pf_rp = rp;
    L->pf_Kl = Kx;
    L->mf_npw = mf_npw;
    L->mf_Kz = mf_Kz;
    L->mf_S = mf_S;
    L->mf_tiles = mf_tiles;
    L->mf_part = o_mfp ? reinterpret_cast<float*>(d + o_mfp) : nullptr;
    L->mf_ooff = o_mfo ? reinterpret_cast<int32_t*>(d + o_mfo) : nullptr;
    L->mf_oent = o_mfe ? reinterpret_cast<uint32_t*>(d + o_mfe) : nullptr;
    L->mf_nzs = o_mfz ? reinterpret_cast<int32_t*>(d + o_mfz) : nullptr;
    L->ws_bytes = off - align256(base);
  }
  if (largest) *largest = big;
  return off;
}

// The kernels address every device buffer through a 32-bit byte range whose
// top half is the "no load" offset, so no buffer may reach 2 GiB: a workspace
// buffer, or the activations of max_M rows.
static bool buffers_fit(const cl_blob_header& h, int32_t max_M) {
  size_t largest = 0;
  workspace_layout(h, max_M, nullptr, h.total_bytes, &largest);
  const size_t xbytes = (size_t)max_M * (size_t)round_up(h.K, 8) * 2;
  return largest < ((size_t)1 << 31) && xbytes < ((size_t)1 << 31);
}

// Host fp16 / bf16 helpers for the prefill's converted copies (round to nearest even).
static float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
static float bf2f(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }
static uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
static uint16_t f2bf(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Host-built inputs of the matrix-core prefill, from the blob: the outlier
// lists per (128-row tile, K step) -- entry = row in tile | k in step << 7 |
// fp16 value << 16, tiles in order, steps in order, rows then columns inside --
// and the rank factors in the MFMA input type (bf16 for bf16 activations, else
// fp16): R^T twice per row [Npad][2 rp], L^T rows padded to Kl = K rounded to 8.
struct PrefillHost {
  std::vector<int32_t> cptr;
  std::vector<uint32_t> cent;
  std::vector<uint16_t> r16, l16;
};
// r16_only: just R^T twice (a bitmap layer: no LDS-tile prefill data).
static void build_prefill_host(const cl_blob_header& h, const uint8_t* b, int Npad, int nd, int rp, int Kl,
                               PrefillHost& out, bool r16_only) {
  const bool bf = h.x_dtype == CL_ACT_BF16;
  auto to16 = [&](float f) { return bf ? f2bf(f) : f2h(f); };
  if (h.nnz > 0 && !r16_only) {
    const int bk = pf_step_k(h.dense, h.mask), tr = pf_tile_rows(h.dense), nt = (int)ceil_div(Npad, tr);
    const int rbits = tr == 256 ? 8 : 7;  // entry: row in tile | k in step << rbits | fp16 value << 16
    const int32_t* rp_ = reinterpret_cast<const int32_t*>(b + h.off[CL_SEC_ROWPTR]);
    const int32_t* col = reinterpret_cast<const int32_t*>(b + h.off[CL_SEC_COL]);
    const uint16_t* val = reinterpret_cast<const uint16_t*>(b + h.off[CL_SEC_VAL]);
    out.cptr.assign((size_t)nt * (nd + 1), 0);
    std::vector<int32_t> cnt((size_t)nt * nd, 0);
    for (int n = 0; n < h.N; ++n)
      for (int p = rp_[n]; p < rp_[n + 1]; ++p) ++cnt[(size_t)(n / tr) * nd + col[p] / bk];
    int32_t acc = 0;
    for (int t = 0; t < nt; ++t) {
      for (int s = 0; s < nd; ++s) {
        out.cptr[(size_t)t * (nd + 1) + s] = acc;
        acc += cnt[(size_t)t * nd + s];
      }
      out.cptr[(size_t)t * (nd + 1) + nd] = acc;
    }
    out.cent.assign((size_t)h.nnz, 0);
    std::vector<int32_t> fill((size_t)nt * nd);
    for (int t = 0; t < nt; ++t)
      for (int s = 0; s < nd; ++s) fill[(size_t)t * nd + s] = out.cptr[(size_t)t * (nd + 1) + s];
    for (int n = 0; n < h.N; ++n)
      for (int p = rp_[n]; p < rp_[n + 1]; ++p) {
        const int s = col[p] / bk;
        out.cent[fill[(size_t)(n / tr) * nd + s]++] =
            (uint32_t)(n % tr) | ((uint32_t)(col[p] - s * bk) << rbits) | ((uint32_t)val[p] << 16);
      }
  }
  if (h.lr != CL_LR_NONE && h.rank > 0) {
    const int r = h.rank, g = h.group > 0 ? h.group : 1;
    const uint8_t* R = b + h.off[CL_SEC_R];
    const uint8_t* Lf = b + h.off[CL_SEC_L];
    const uint16_t* Rs = reinterpret_cast<const uint16_t*>(b + h.off[CL_SEC_RSCALE]);
    const uint16_t* Ls = reinterpret_cast<const uint16_t*>(b + h.off[CL_SEC_LSCALE]);
    auto factor = [&](const uint8_t* F, const uint16_t* S, int row, int j, int len) -> float {
      if (h.lr == CL_LR_INT4) {
        const int q = (int)((F[(size_t)row * ((len + 1) / 2) + j / 2] >> (4 * (j & 1))) & 0xF) - 8;
        return (float)q * h2f(S[(size_t)row * ceil_div(len, g) + j / g]);
      }
      const uint16_t u = reinterpret_cast<const uint16_t*>(F)[(size_t)row * len + j];
      return h.lr == CL_LR_BF16 ? bf2f(u) : h2f(u);
    };
    out.r16.assign((size_t)Npad * 2 * rp, 0);
    for (int n = 0; n < Npad; ++n)
      for (int j = 0; j < r; ++j) {
        const uint16_t v = to16(factor(R, Rs, n, j, r));
        out.r16[(size_t)n * 2 * rp + j] = v;
        out.r16[(size_t)n * 2 * rp + rp + j] = v;
      }
    if (r16_only) return;
    out.l16.assign((size_t)r * Kl, 0);
    for (int j = 0; j < r; ++j)
      for (int k = 0; k < h.K; ++k) out.l16[(size_t)j * Kl + k] = to16(factor(Lf, Ls, j, k, h.K));
  }
}

// Outlier lists of the matrix-core decode: the CSR entries regrouped by
// (K slice z, 128-row tile, row in tile) -- list index (z * tiles + tile) * 128
// + row -- each list in ascending column order, entry = column - z * Kz (low 16
// bits) | fp16 value << 16.
static void build_mfma_outliers(const cl_blob_header& h, const uint8_t* b, int S, int tiles, int Kz,
                                std::vector<int32_t>& off, std::vector<uint32_t>& ent) {
  const int32_t* rp = reinterpret_cast<const int32_t*>(b + h.off[CL_SEC_ROWPTR]);
  const int32_t* col = reinterpret_cast<const int32_t*>(b + h.off[CL_SEC_COL]);
  const uint16_t* val = reinterpret_cast<const uint16_t*>(b + h.off[CL_SEC_VAL]);
  off.assign((size_t)S * tiles * kMfRows + 1, 0);
  auto list = [&](int n, int c) { return ((size_t)(c / Kz) * tiles + n / kMfRows) * kMfRows + n % kMfRows; };
  for (int n = 0; n < h.N; ++n)
    for (int p = rp[n]; p < rp[n + 1]; ++p) ++off[list(n, col[p]) + 1];
  for (size_t i = 1; i < off.size(); ++i) off[i] += off[i - 1];
  std::vector<int32_t> fill(off.begin(), off.end() - 1);
  ent.assign((size_t)h.nnz, 0);
  for (int n = 0; n < h.N; ++n)
    for (int p = rp[n]; p < rp[n + 1]; ++p) {
      const int c = col[p];
      ent[fill[list(n, c)]++] = (uint32_t)(c % Kz) | ((uint32_t)val[p] << 16);
    }
}

// The decode prologue's copy of L from the blob's L^T: k-major, two consecutive
// k per (pair, column) -- 16-bit: [Kl/2][rpad][2] values; int4: [Kl/2][rpad]
// bytes, k even in the low nibble, codes as stored (zero padding is code 8) --
// and the int4 scales k-major [ceil(Kl/group)][rpad].  Kl = slices * kLrSlice.
static void build_lowrank_host(const cl_blob_header& h, const uint8_t* b, int mode, int rpad, int S,
                               std::vector<uint8_t>& lk, std::vector<uint16_t>& ls) {
  const int r = h.rank, K = h.K;
  const size_t Kl = (size_t)S * kLrSlice;
  const uint8_t* Lf = b + h.off[CL_SEC_L];
  if (mode == 0) {
    lk.assign(Kl * rpad * 2, 0);
    uint16_t* o = reinterpret_cast<uint16_t*>(lk.data());
    const uint16_t* src = reinterpret_cast<const uint16_t*>(Lf);
    for (int j = 0; j < r; ++j)
      for (int k = 0; k < K; ++k) o[((size_t)(k >> 1) * rpad + j) * 2 + (k & 1)] = src[(size_t)j * K + k];
    return;
  }
  const int g = h.group, hk = (K + 1) / 2, gk = (int)ceil_div(K, g);
  lk.assign(Kl / 2 * rpad, 0x88);
  for (int j = 0; j < r; ++j)
    for (int k = 0; k < K; ++k) {
      const uint8_t c = (Lf[(size_t)j * hk + k / 2] >> (4 * (k & 1))) & 0xF;
      uint8_t& d = lk[(size_t)(k >> 1) * rpad + j];
      d = (uint8_t)((d & (0xF0 >> (4 * (k & 1)))) | (c << (4 * (k & 1))));
    }
  const uint16_t* Ls = reinterpret_cast<const uint16_t*>(b + h.off[CL_SEC_LSCALE]);
  ls.assign((size_t)ceil_div(Kl, g) * rpad, 0);
  for (int j = 0; j < r; ++j)
    for (int q = 0; q < gk; ++q) ls[(size_t)q * rpad + j] = Ls[(size_t)j * gk + q];
}

static void destroy_layer(Layer* L) {
  if (!L) return;
  if (L->wait_err_host) (void)hipHostFree(const_cast<uint32_t*>(L->wait_err_host));
  delete L;
}

template <class T>
static T* sec(uint8_t* dev, const cl_blob_header& h, int s) {
  return h.len[s] ? reinterpret_cast<T*>(dev + h.off[s]) : nullptr;
}

}  // namespace cl

using namespace cl;

extern "C" size_t cl_device_bytes(const void* blob, int32_t max_M) {
  const cl_blob_header* h;
  if (max_M < 1 || check_blob(blob, &h) != CL_OK) return 0;
  if (!buffers_fit(*h, max_M)) {
    fail(CL_ESIZE, "a workspace buffer or the activations of max_M rows would reach 2 GiB");
    return 0;
  }
  return workspace_layout(*h, max_M, nullptr, h->total_bytes);
}

extern "C" cl_status cl_create(const void* blob, void* dev_buf, size_t dev_bytes, int32_t max_M, void* stream,
                               void** handle) {
  clear_error();
  if (!handle) return fail(CL_EINVAL, "handle is NULL");
  *handle = nullptr;
  const cl_blob_header* h;
  cl_status st = check_blob(blob, &h);
  if (st != CL_OK) return st;
  if (max_M < 1) return fail(CL_EINVAL, "max_M must be >= 1");
  if (!buffers_fit(*h, max_M)) return fail(CL_ESIZE, "a workspace buffer or the activations of max_M rows would reach 2 GiB");
  if (!dev_buf || reinterpret_cast<uintptr_t>(dev_buf) % 256) return fail(CL_EINVAL, "dev_buf must be 256-byte aligned");
  if (h->lr != CL_LR_NONE && h->rank > 256) return fail(CL_EUNSUPPORTED, "ranks above 256 are not built");
  Layer* L = new (std::nothrow) Layer();
  if (!L) return fail(CL_EINVAL, "out of host memory");
  L->h = *h;
  L->dev = static_cast<uint8_t*>(dev_buf);
  L->max_M = max_M;
  L->Npad = h->n_tiles * 64;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int cus = 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  L->num_cus = cus;
  L->split = choose_split(*h, cus);
  L->wait_polls = kLrMaxPolls;
  {  // the error word of the waits for t, in pinned host memory mapped for the device
    void* hp = nullptr;
    void* dp = nullptr;
    hipError_t he = hipHostMalloc(&hp, 64, hipHostMallocMapped);
    if (he == hipSuccess) he = hipHostGetDevicePointer(&dp, hp, 0);
    if (he != hipSuccess) {
      if (hp) (void)hipHostFree(hp);
      delete L;
      return fail(CL_EHIP, "pinned error word: %s", hipGetErrorString(he));
    }
    L->wait_err_host = static_cast<volatile uint32_t*>(hp);
    L->wait_err_host[0] = 0;
    L->wait_err_dev = static_cast<uint32_t*>(dp);
  }
  const size_t need = workspace_layout(*h, max_M, L, h->total_bytes);
  if (dev_bytes < need) {
    destroy_layer(L);
    return fail(CL_ENOMEM, "dev_buf needs %zu bytes, got %zu", need, dev_bytes);
  }
  L->dev_bytes = dev_bytes;
  uint8_t* d = L->dev;
  L->dense = sec<uint8_t>(d, *h, CL_SEC_DENSE);
  L->table = sec<uint8_t>(d, *h, CL_SEC_TABLE);
  L->xscale = h->n_xscale > 0 ? sec<uint16_t>(d, *h, CL_SEC_XSCALE) : nullptr;
  L->meta = sec<uint8_t>(d, *h, CL_SEC_META);
  L->nzoff = sec<int32_t>(d, *h, CL_SEC_NZOFF);
  L->rowptr = sec<int32_t>(d, *h, CL_SEC_ROWPTR);
  L->col = sec<int32_t>(d, *h, CL_SEC_COL);
  L->val = sec<uint16_t>(d, *h, CL_SEC_VAL);
  L->L = sec<uint8_t>(d, *h, CL_SEC_L);
  L->R = sec<uint8_t>(d, *h, CL_SEC_R);
  L->Lscale = sec<uint16_t>(d, *h, CL_SEC_LSCALE);
  L->Rscale = sec<uint16_t>(d, *h, CL_SEC_RSCALE);
  hipStream_t s = static_cast<hipStream_t>(stream);

  // bitmap: byte offset of the first kept value of every wave slice of every row
  std::vector<int32_t> nzs;
  if (h->mask == CL_MASK_BITMAP) {
    const int nsl = 4 * L->split;
    nzs.assign((size_t)L->Npad * nsl, 0);
    const uint8_t* b = static_cast<const uint8_t*>(blob);
    const int32_t* off = reinterpret_cast<const int32_t*>(b + h->off[CL_SEC_NZOFF]);
    const uint32_t* meta = reinterpret_cast<const uint32_t*>(b + h->off[CL_SEC_META]);
    for (int n = 0; n < h->N; ++n) {
      long long cnt = 0;
      int c = 0;
      for (int q = 0; q < nsl; ++q) {
        const int cb = (int)((long long)h->chunks * q / nsl);
        for (; c < cb; ++c) {
          const uint32_t* w = meta + ((size_t)n * h->chunks + c) * 4;
          cnt += __builtin_popcount(w[0]) + __builtin_popcount(w[1]) + __builtin_popcount(w[2]) + __builtin_popcount(w[3]);
        }
        nzs[(size_t)n * nsl + q] = (int32_t)(off[n] + cnt);
      }
    }
  }
  // batch 1: the streaming kernel's plan (its outlier capacity from the row pointers)
  L->st = plan_stream(*h, h->nnz > 0 ? reinterpret_cast<const int32_t*>(static_cast<const uint8_t*>(blob) + h->off[CL_SEC_ROWPTR])
                                     : nullptr,
                      L->num_cus, L->lr_mode);
  PrefillHost pf;
  const bool bm_pf = L->pf_dense8 != nullptr;
  if (h->mask != CL_MASK_BITMAP || bm_pf || L->pf_r16)
    build_prefill_host(*h, static_cast<const uint8_t*>(blob), L->Npad, L->pf_nd, L->pf_rp, L->pf_Kl, pf,
                       h->mask == CL_MASK_BITMAP && !bm_pf);
  // bitmap layer for prefill: the dense INT8 chunk stream (u = q + 128, 16 k per
  // chunk, rows of pf_chunks8 chunks; 128 = zero for dropped weights and padding)
  std::vector<uint8_t> d8;
  if (bm_pf) {
    d8.assign((size_t)L->Npad * L->pf_chunks8 * 16, 128u);
    const uint8_t* b = static_cast<const uint8_t*>(blob);
    const int32_t* off = reinterpret_cast<const int32_t*>(b + h->off[CL_SEC_NZOFF]);
    const uint32_t* meta = reinterpret_cast<const uint32_t*>(b + h->off[CL_SEC_META]);
    const int8_t* kept = reinterpret_cast<const int8_t*>(b + h->off[CL_SEC_DENSE]);
    for (int n = 0; n < h->N; ++n) {
      long long p = off[n];
      uint8_t* row = d8.data() + (size_t)n * L->pf_chunks8 * 16;
      for (int c = 0; c < h->chunks; ++c) {
        const uint32_t* w = meta + ((size_t)n * h->chunks + c) * 4;
        for (int t = 0; t < 128; ++t)
          if ((w[t >> 5] >> (t & 31)) & 1u) row[128 * c + t] = (uint8_t)(kept[p++] + 128);
      }
    }
  }
  std::vector<int32_t> mfo;
  std::vector<uint32_t> mfe;
  // bitmap, matrix-core decode: first kept byte of every (row, K slice)
  std::vector<int32_t> mfz;
  if (L->mf_nzs) {
    const uint8_t* b = static_cast<const uint8_t*>(blob);
    const int32_t* off = reinterpret_cast<const int32_t*>(b + h->off[CL_SEC_NZOFF]);
    const uint32_t* meta = reinterpret_cast<const uint32_t*>(b + h->off[CL_SEC_META]);
    const int cps = L->mf_Kz / h->span;  // chunks per slice
    mfz.assign((size_t)L->Npad * L->mf_S, 0);
    for (int n = 0; n < h->N; ++n) {
      long long cnt = off[n];
      for (int zz = 0; zz < L->mf_S; ++zz) {
        mfz[(size_t)n * L->mf_S + zz] = (int32_t)cnt;
        for (int c = zz * cps; c < (zz + 1) * cps && c < h->chunks; ++c) {
          const uint32_t* w = meta + ((size_t)n * h->chunks + c) * 4;
          cnt += __builtin_popcount(w[0]) + __builtin_popcount(w[1]) + __builtin_popcount(w[2]) + __builtin_popcount(w[3]);
        }
      }
    }
  }
  if (L->mf_ooff)
    build_mfma_outliers(*h, static_cast<const uint8_t*>(blob), L->mf_S, L->mf_tiles, L->mf_Kz, mfo, mfe);
  std::vector<uint8_t> lrk;
  std::vector<uint16_t> lrs;
  if (L->lr_mode >= 0)
    build_lowrank_host(*h, static_cast<const uint8_t*>(blob), L->lr_mode, L->lr_rpad, L->lr_S, lrk, lrs);
  hipError_t e = hipMemcpyAsync(d, blob, h->total_bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !lrk.empty()) e = hipMemcpyAsync(L->lr_lk, lrk.data(), lrk.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !lrs.empty()) e = hipMemcpyAsync(L->lr_ls, lrs.data(), lrs.size() * 2, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && L->lr_cnt) e = hipMemsetAsync(L->lr_cnt, 0, kLrCntWords * 4, s);
  // the tagged partial sums of t: tag 0 matches no launch (epochs start at 1,
  // recorded launches carry the top bit), so words that an earlier layer left
  // in this memory cannot pass for this layer's
  if (e == hipSuccess && L->lr_part) e = hipMemsetAsync(L->lr_part, 0, L->lr_part_bytes, s);
  if (e == hipSuccess) e = hipMemsetAsync(L->counters, 0, (size_t)(h->n_tiles + ceil_div(max_M, 32) + 8) * 4, s);
  if (e == hipSuccess && !nzs.empty())
    e = hipMemcpyAsync(L->nzstart, nzs.data(), nzs.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !d8.empty()) e = hipMemcpyAsync(L->pf_dense8, d8.data(), d8.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !pf.cptr.empty())
    e = hipMemcpyAsync(L->pf_cptr, pf.cptr.data(), pf.cptr.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !pf.cent.empty())
    e = hipMemcpyAsync(L->pf_cent, pf.cent.data(), pf.cent.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !pf.r16.empty())
    e = hipMemcpyAsync(L->pf_r16, pf.r16.data(), pf.r16.size() * 2, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !pf.l16.empty())
    e = hipMemcpyAsync(L->pf_l16, pf.l16.data(), pf.l16.size() * 2, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !mfz.empty())
    e = hipMemcpyAsync(L->mf_nzs, mfz.data(), mfz.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !mfo.empty())
    e = hipMemcpyAsync(L->mf_ooff, mfo.data(), mfo.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !mfe.empty())
    e = hipMemcpyAsync(L->mf_oent, mfe.data(), mfe.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    destroy_layer(L);
    return fail(CL_EHIP, "upload failed: %s", hipGetErrorString(e));
  }
  *handle = L;
  return CL_OK;
}

static cl_status forward_impl(Layer* L, int32_t M, const void* x, float* y, void* stream, int32_t path) {
  if (!L) return fail(CL_EINVAL, "handle is NULL");
  if (M < 1 || M > L->max_M) return fail(CL_EINVAL, "M=%d outside [1, %d]", M, L->max_M);
  if (!x || !y) return fail(CL_EINVAL, "x or y is NULL");
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(y) % 16)
    return fail(CL_EINVAL, "x and y must be 16-byte aligned");
  if (path == CL_PATH_AUTO) path = M <= kMaxDecodeM ? CL_PATH_DECODE : CL_PATH_PREFILL;
  if (path != CL_PATH_DECODE && path != CL_PATH_PREFILL && path != CL_PATH_DECODE_VALU &&
      path != CL_PATH_DECODE_MFMA && path != CL_PATH_DECODE_STREAM)
    return fail(CL_EINVAL, "unknown path %d", path);
  const bool decode = path != CL_PATH_PREFILL;
  if (decode && M > kMaxDecodeM) return fail(CL_EINVAL, "the decode path takes M <= %d", kMaxDecodeM);
  if (path == CL_PATH_DECODE_MFMA && L->mf_S == 0)
    return fail(CL_EUNSUPPORTED, "the matrix-core decode needs a bitmap layer or one created with max_M >= 2");
  if (path == CL_PATH_DECODE_STREAM && (M != 1 || !L->st.ok))
    return fail(CL_EUNSUPPORTED, "the streaming decode takes M = 1 and a layer that fits its LDS plan");
  if (L->wait_err_host && L->wait_err_host[0]) {  // set by a wait for t that gave up in an earlier forward
    L->wait_err_host[0] = 0;
    return fail(CL_EHIP, "an earlier forward on this layer gave up waiting for x' L inside its launch; "
                         "its outputs hold NaN (reported once; this call did nothing)");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (decode) {  // the decode dispatch clamps / restages x itself (in its kernels where it can)
    const int variant = path == CL_PATH_DECODE_VALU ? 1 : path == CL_PATH_DECODE_MFMA ? 2
                      : path == CL_PATH_DECODE_STREAM ? 3 : 0;
    e = launch_decode(*L, M, x, y, s, variant);
  } else {
    const void* xa = x;
    if (L->xprep) {
      e = launch_prep_x(*L, M, x, s);
      xa = L->xprep;
    }
    if (e == hipSuccess) e = launch_prefill(*L, M, xa, y, s);
  }
  if (e != hipSuccess) return fail(CL_EHIP, "launch failed: %s", hipGetErrorString(e));
  return CL_OK;
}

extern "C" cl_status cl_forward(void* handle, int32_t M, const void* x_dev, float* y_dev, void* stream) {
  clear_error();
  return forward_impl(static_cast<Layer*>(handle), M, x_dev, y_dev, stream, CL_PATH_AUTO);
}

extern "C" cl_status cl_forward_path(void* handle, int32_t M, const void* x_dev, float* y_dev, void* stream,
                                     int32_t path) {
  clear_error();
  return forward_impl(static_cast<Layer*>(handle), M, x_dev, y_dev, stream, path);
}

extern "C" cl_status cl_debug_dequant(void* handle, uint16_t* D16, uint16_t* S16, float* L32, float* R32,
                                      void* stream) {
  clear_error();
  Layer* L = static_cast<Layer*>(handle);
  if (!L) return fail(CL_EINVAL, "handle is NULL");
  if (!D16 || !S16) return fail(CL_EINVAL, "D16 and S16 are required");
  hipError_t e = launch_debug(*L, D16, S16, L32, R32, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(CL_EHIP, "debug launch failed: %s", hipGetErrorString(e));
  return CL_OK;
}

extern "C" cl_status cl_destroy(void* handle) {
  clear_error();
  destroy_layer(static_cast<Layer*>(handle));
  return CL_OK;
}

extern "C" cl_status cl_set_wait_limit(void* handle, uint32_t max_polls, int32_t withhold) {
  clear_error();
  Layer* L = static_cast<Layer*>(handle);
  if (!L) return fail(CL_EINVAL, "handle is NULL");
  L->wait_polls = max_polls;
  L->wait_withhold = withhold ? 1 : 0;
  return CL_OK;
}
