// pack.cpp -- host packer: validates a logical layer and lays it out for the GPU.
//
// Host only (no HIP calls), so the whole packer is testable on a CPU.
// Format sources:
//   "SqueezeLLM: Dense-and-Sparse Quantization", Approach: per-weight LUT
//     codes and a full-precision CSR matrix of outliers;
//   "SLiM: One-shot Quantization and Sparsity with Low-rank Approximation for
//     LLM Weight Compression", review highlights and rebuttal: symmetric
//     integer weights, 2:4 or unstructured masks, low-rank adapters with
//     AbsMax int4 groups of 128;
//   "Compressing Large Language Models by Joint Sparsification and
//     Quantization", Approach: unstructured sparsity with quantization and a
//     per-layer activation clamp.
// The device layout of each section is described in layout.h.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "internal.h"
#include "layout.h"

namespace cl {

static thread_local std::string g_err;

cl_status fail(cl_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

void clear_error() { g_err.clear(); }

// Largest section or device buffer: the kernels address every buffer through
// a hardware-checked 32-bit byte range whose top half is the "no load" offset.
constexpr uint64_t kMaxBufferBytes = (uint64_t)1 << 31;

// Section lengths a header implies (the bitmap's DENSE length depends on its
// kept counts and is checked against NZOFF instead; returned as 0 here).
static void expected_lengths(const cl_blob_header* h, uint64_t len[CL_SEC_COUNT]) {
  const KindInfo ki = kind_info(h->dense, h->mask);
  const uint64_t N = (uint64_t)h->N, K = (uint64_t)h->K, Npad = (uint64_t)h->n_tiles * kTileRows;
  const uint64_t C = (uint64_t)h->chunks, r = (uint64_t)h->rank, g = h->group > 0 ? (uint64_t)h->group : 1;
  for (int s = 0; s < CL_SEC_COUNT; ++s) len[s] = 0;
  const bool bitmap = h->mask == CL_MASK_BITMAP;
  if (!bitmap) len[CL_SEC_DENSE] = Npad * C * kChunkBytes;
  if (ki.meta_chunk_bytes) len[CL_SEC_META] = Npad * C * (uint64_t)ki.meta_chunk_bytes;
  if (bitmap) len[CL_SEC_NZOFF] = (N + 1) * 4;
  len[CL_SEC_TABLE] = ki.table_entries ? Npad * (uint64_t)ki.table_entries * 2 : Npad * 2;
  if (h->nnz > 0) {
    len[CL_SEC_ROWPTR] = (N + 1) * 4;
    len[CL_SEC_COL] = (uint64_t)h->nnz * 4;
    len[CL_SEC_VAL] = (uint64_t)h->nnz * 2;
  }
  if (h->lr != CL_LR_NONE) {
    if (h->lr == CL_LR_INT4) {
      len[CL_SEC_L] = r * ((K + 1) / 2);
      len[CL_SEC_R] = Npad * ((r + 1) / 2);
      len[CL_SEC_LSCALE] = (uint64_t)ceil_div((int64_t)K, (int64_t)g) * r * 2;
      len[CL_SEC_RSCALE] = (uint64_t)ceil_div((int64_t)r, (int64_t)g) * Npad * 2;
    } else {
      len[CL_SEC_L] = K * r * 2;
      len[CL_SEC_R] = r * Npad * 2;
    }
  }
  if (h->n_xscale > 0) len[CL_SEC_XSCALE] = K * 2;
}

// A blob is trusted by cl_create and the kernels only after this check: the
// header fields agree with each other, every section has the length the
// header implies and lies inside total_bytes (overflow-safe), no section
// reaches 2 GiB, and the contents the host and the kernels index with are in
// range -- CSR row pointers and columns, the bitmap's row offsets against its
// keep bits, zero keep bits on the padding rows.  The blob must hold
// total_bytes bytes (a blob from cl_pack does).
cl_status check_blob(const void* blob, const cl_blob_header** out) {
  if (!blob) return fail(CL_EINVAL, "blob is NULL");
  if (reinterpret_cast<uintptr_t>(blob) % 8) return fail(CL_EINVAL, "blob is not 8-byte aligned");
  const cl_blob_header* h = static_cast<const cl_blob_header*>(blob);
  if (h->magic != CL_BLOB_MAGIC || h->version != CL_BLOB_VERSION)
    return fail(CL_EINVAL, "not a compressed-linear blob (magic/version)");
  if (h->K < 1 || h->N < 1 || h->K > (1 << 24) || h->N > (1 << 24) || h->n_tiles != (int32_t)ceil_div(h->N, kTileRows))
    return fail(CL_EINVAL, "blob header has inconsistent dimensions");
  const KindInfo ki = kind_info(h->dense, h->mask);
  if (ki.span == 0 || ki.span != h->span || h->chunks != (int32_t)ceil_div(h->K, ki.span) ||
      h->meta_chunk_bytes != ki.meta_chunk_bytes)
    return fail(CL_EINVAL, "blob header has an unknown or inconsistent format");
  if (h->lr < CL_LR_NONE || h->lr > CL_LR_INT4 || (h->lr == CL_LR_NONE) != (h->rank == 0) || h->rank < 0 ||
      h->rank > 4096 || (h->lr == CL_LR_INT4 ? h->group < 1 : h->group != 0))
    return fail(CL_EINVAL, "blob header has an inconsistent low-rank part");
  if ((h->x_dtype != CL_ACT_F16 && h->x_dtype != CL_ACT_BF16) || (h->has_clamp != 0 && h->has_clamp != 1))
    return fail(CL_EINVAL, "blob header has an unknown activation type or clamp flag");
  if (h->nnz < 0 || h->nnz > 0x7FFFFFFFLL) return fail(CL_EINVAL, "blob header has nnz out of range");
  if (h->n_xscale < 0 || h->n_xscale > h->K) return fail(CL_EINVAL, "blob header has an inconsistent activation-scale section");
  if (h->total_bytes < sizeof(cl_blob_header)) return fail(CL_EINVAL, "blob header has total_bytes below the header");
  uint64_t want[CL_SEC_COUNT];
  expected_lengths(h, want);
  for (int s = 0; s < CL_SEC_COUNT; ++s) {
    const uint64_t len = h->len[s], off = h->off[s];
    if (len >= kMaxBufferBytes) return fail(CL_ESIZE, "blob section %d holds 2 GiB or more", s);
    if (len && (off % 256 || off < sizeof(cl_blob_header) || len > h->total_bytes || off > h->total_bytes - len))
      return fail(CL_EINVAL, "blob section %d lies outside the blob", s);
    const bool dense_bm = s == CL_SEC_DENSE && h->mask == CL_MASK_BITMAP;
    if (!dense_bm && len != want[s])
      return fail(CL_EINVAL, "blob section %d has %llu bytes, the header implies %llu", s, (unsigned long long)len,
                  (unsigned long long)want[s]);
  }
  const uint8_t* b = static_cast<const uint8_t*>(blob);
  if (h->nnz > 0) {
    const int32_t* rp = reinterpret_cast<const int32_t*>(b + h->off[CL_SEC_ROWPTR]);
    const int32_t* col = reinterpret_cast<const int32_t*>(b + h->off[CL_SEC_COL]);
    if (rp[0] != 0 || (int64_t)rp[h->N] != h->nnz) return fail(CL_EINVAL, "blob CSR row pointers do not run from 0 to nnz");
    for (int64_t n = 0; n < h->N; ++n) {
      if (rp[n + 1] < rp[n]) return fail(CL_EINVAL, "blob CSR row pointers decrease at row %lld", (long long)n);
      for (int64_t p = rp[n]; p < rp[n + 1]; ++p)
        if (col[p] < 0 || col[p] >= h->K || (p > rp[n] && col[p] <= col[p - 1]))
          return fail(CL_EINVAL, "blob CSR columns of row %lld are out of range or not increasing", (long long)n);
    }
  }
  if (h->mask == CL_MASK_BITMAP) {
    const int32_t* off = reinterpret_cast<const int32_t*>(b + h->off[CL_SEC_NZOFF]);
    const uint32_t* meta = reinterpret_cast<const uint32_t*>(b + h->off[CL_SEC_META]);
    const int64_t C = h->chunks, Npad = (int64_t)h->n_tiles * kTileRows;
    if (off[0] != 0) return fail(CL_EINVAL, "blob bitmap offsets do not start at 0");
    for (int64_t n = 0; n < Npad; ++n) {
      int64_t kept = 0;
      for (int64_t i = 0; i < C * 4; ++i) kept += __builtin_popcount(meta[n * C * 4 + i]);
      if (n >= h->N) {
        if (kept) return fail(CL_EINVAL, "blob bitmap keeps weights on padding row %lld", (long long)n);
        continue;
      }
      if (off[n] % 16 || (int64_t)off[n + 1] - (int64_t)off[n] < kept)
        return fail(CL_EINVAL, "blob bitmap offsets of row %lld do not hold its kept values", (long long)n);
    }
    if ((uint64_t)off[h->N] + 64 > h->len[CL_SEC_DENSE])
      return fail(CL_EINVAL, "blob bitmap values run past their section");
  }
  if (out) *out = h;
  return CL_OK;
}

namespace {

inline bool f16_is_finite_nonneg(uint16_t b) { return !(b & 0x8000u) && ((b >> 10) & 0x1F) != 0x1F; }

struct Plan {
  int64_t K, N, n_tiles, Npad, chunks, span, meta_cb, tab_entries;
  int64_t nnz, rank, group, lr_half_r;
  uint64_t off[CL_SEC_COUNT] = {}, len[CL_SEC_COUNT] = {};
  uint64_t total = 0;
  std::vector<int64_t> nz_count;  // BITMAP: kept per row
  std::vector<int64_t> nz_off;    // BITMAP: device start of each row (16-aligned)
  cl_bytes acct = {};
};

cl_status validate(const cl_layer_desc* d) {
  if (!d) return fail(CL_EINVAL, "desc is NULL");
  if (d->K < 1 || d->N < 1) return fail(CL_EINVAL, "K and N must be >= 1 (K=%d N=%d)", d->K, d->N);
  if (d->K > (1 << 24) || d->N > (1 << 24)) return fail(CL_ESIZE, "K and N must be <= 2^24");
  if (d->dense < 0 || d->dense > 3) return fail(CL_EINVAL, "unknown dense kind %d", d->dense);
  if (d->mask < 0 || d->mask > 2) return fail(CL_EINVAL, "unknown mask kind %d", d->mask);
  if (d->lr < 0 || d->lr > 3) return fail(CL_EINVAL, "unknown low-rank kind %d", d->lr);
  if (d->x_dtype != CL_ACT_F16 && d->x_dtype != CL_ACT_BF16) return fail(CL_EINVAL, "unknown x dtype %d", d->x_dtype);
  const bool lut = d->dense <= CL_DENSE_LUT4;
  if (lut && d->mask != CL_MASK_NONE) return fail(CL_EUNSUPPORTED, "masks are built for the integer formats only");
  if (d->dense == CL_DENSE_INT4 && d->mask == CL_MASK_BITMAP)
    return fail(CL_EUNSUPPORTED, "the bitmap mask is built for INT8 values");
  if (d->dense == CL_DENSE_INT8 && d->mask == CL_MASK_2_4)
    return fail(CL_EUNSUPPORTED, "the 2:4 mask is built for INT4 values");
  if (d->mask == CL_MASK_2_4 && d->K % 4) return fail(CL_EUNSUPPORTED, "2:4 needs K %% 4 == 0 (K=%d)", d->K);
  const int64_t K = d->K, N = d->N;
  {  // sizes first (from the dimensions alone, before any array is read): no section may reach 2 GiB
    cl_blob_header hd = {};
    hd.K = d->K;
    hd.N = d->N;
    hd.dense = d->dense;
    hd.mask = d->mask;
    hd.n_tiles = (int32_t)ceil_div(N, kTileRows);
    hd.chunks = (int32_t)ceil_div(K, kind_info(d->dense, d->mask).span);
    hd.lr = d->rank > 0 ? d->lr : CL_LR_NONE;
    hd.rank = d->lr != CL_LR_NONE && d->rank > 0 ? d->rank : 0;
    hd.group = d->group > 0 ? d->group : 1;
    hd.nnz = d->nnz > 0 ? d->nnz : 0;
    hd.n_xscale = d->n_xscale > 0 ? 1 : 0;
    uint64_t len[CL_SEC_COUNT];
    expected_lengths(&hd, len);
    // (the bitmap's kept values are counted, and checked, once the mask is read)
    for (int sct = 0; sct < CL_SEC_COUNT; ++sct)
      if (len[sct] >= kMaxBufferBytes)
        return fail(CL_ESIZE, "section %d of the device layout would hold %llu bytes (at most 2^31 - 1)", sct,
                    (unsigned long long)len[sct]);
  }
  if (lut) {
    if (!d->codes || !d->lut) return fail(CL_EINVAL, "LUT formats need codes and lut");
    const int nb = d->dense == CL_DENSE_LUT3 ? 8 : 16;
    for (int64_t i = 0; i < N * K; ++i)
      if (d->codes[i] >= nb) return fail(CL_EINVAL, "code %d out of range at %lld", d->codes[i], (long long)i);
  } else {
    if (!d->qvals || !d->row_scale) return fail(CL_EINVAL, "integer formats need qvals and row_scale");
    const int lo = d->dense == CL_DENSE_INT4 ? -8 : -127, hi = d->dense == CL_DENSE_INT4 ? 7 : 127;
    if (d->mask != CL_MASK_NONE && !d->keep) return fail(CL_EINVAL, "a mask needs keep");
    for (int64_t i = 0; i < N * K; ++i) {
      const bool kept = d->mask == CL_MASK_NONE || d->keep[i];
      if (d->mask != CL_MASK_NONE && d->keep[i] > 1) return fail(CL_EINVAL, "keep must be 0 or 1 (at %lld)", (long long)i);
      if (kept && (d->qvals[i] < lo || d->qvals[i] > hi))
        return fail(CL_EINVAL, "value %d out of range [%d,%d] at %lld", d->qvals[i], lo, hi, (long long)i);
    }
    if (d->mask == CL_MASK_2_4) {
      for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < K / 4; ++g) {
          const uint8_t* kp = d->keep + n * K + 4 * g;
          if (kp[0] + kp[1] + kp[2] + kp[3] != 2)
            return fail(CL_EINVAL, "2:4 group (row %lld, k %lld) does not keep exactly two", (long long)n, (long long)(4 * g));
        }
    }
  }
  if (d->nnz < 0 || d->nnz > 0x7FFFFFFFLL) return fail(CL_ESIZE, "nnz out of range");
  if (d->nnz > 0) {
    if (!d->csr_row_ptr || !d->csr_col || !d->csr_val) return fail(CL_EINVAL, "CSR arrays are NULL");
    if (d->csr_row_ptr[0] != 0 || d->csr_row_ptr[N] != d->nnz)
      return fail(CL_EINVAL, "CSR row_ptr must start at 0 and end at nnz");
    for (int64_t n = 0; n < N; ++n) {
      const int64_t a = d->csr_row_ptr[n], b = d->csr_row_ptr[n + 1];
      if (b < a) return fail(CL_EINVAL, "CSR row_ptr decreases at row %lld", (long long)n);
      for (int64_t p = a; p < b; ++p) {
        const int32_t c = d->csr_col[p];
        if (c < 0 || c >= K) return fail(CL_EINVAL, "CSR column %d out of range in row %lld", c, (long long)n);
        if (p > a && c <= d->csr_col[p - 1])
          return fail(CL_EINVAL, "CSR columns of row %lld are not strictly increasing", (long long)n);
      }
    }
  }
  if (d->lr != CL_LR_NONE && d->rank > 0) {
    if (d->rank > 4096) return fail(CL_ESIZE, "rank above 4096");
    if (!d->L || !d->R) return fail(CL_EINVAL, "low-rank factors are NULL");
    if (d->lr == CL_LR_INT4) {
      if (d->group < 1) return fail(CL_EINVAL, "int4 low-rank needs group >= 1");
      if (!d->L_scale || !d->R_scale) return fail(CL_EINVAL, "int4 low-rank needs scales");
      const int8_t* L = static_cast<const int8_t*>(d->L);
      const int8_t* R = static_cast<const int8_t*>(d->R);
      for (int64_t i = 0; i < K * d->rank; ++i)
        if (L[i] < -8 || L[i] > 7) return fail(CL_EINVAL, "L code out of range");
      for (int64_t i = 0; i < (int64_t)d->rank * N; ++i)
        if (R[i] < -8 || R[i] > 7) return fail(CL_EINVAL, "R code out of range");
    }
  } else if (d->rank < 0) {
    return fail(CL_EINVAL, "rank must be >= 0");
  }
  if (d->has_clamp && !f16_is_finite_nonneg(d->act_clamp))
    return fail(CL_EINVAL, "the clamp must be a finite, non-negative fp16 value");
  if (d->has_clamp && d->x_dtype == CL_ACT_BF16) {
    // the clamped activation -c / c must be exact in bf16 (8-bit significand)
    const uint32_t e = (d->act_clamp >> 10) & 0x1F, m = d->act_clamp & 0x3FF;
    if (e != 0 && (m & 7u)) return fail(CL_EUNSUPPORTED, "the clamp value is not representable in bf16");
    if (e == 0 && m && (m >> __builtin_ctz(m)) > 0xFF) return fail(CL_EUNSUPPORTED, "the clamp value is not representable in bf16");
  }
  if (d->n_xscale < 0 || d->n_xscale > d->K) return fail(CL_EINVAL, "n_xscale must be in [0, K]");
  if (d->n_xscale > 0) {
    if (!d->xscale_ch || !d->xscale) return fail(CL_EINVAL, "activation scaling arrays are NULL");
    for (int32_t i = 0; i < d->n_xscale; ++i) {
      const int32_t c = d->xscale_ch[i];
      if (c < 0 || c >= d->K) return fail(CL_EINVAL, "scaled channel %d out of range", c);
      if (i > 0 && c <= d->xscale_ch[i - 1]) return fail(CL_EINVAL, "scaled channels are not strictly increasing");
      // a normal fp16 in [2^-14, 1]: x * f is then exact in fp32 and cannot overflow
      if (d->xscale[i] < 0x0400u || d->xscale[i] > 0x3C00u)
        return fail(CL_EINVAL, "activation factor 0x%04x of channel %d is not a normal value in [2^-14, 1]",
                    d->xscale[i], c);
    }
  }
  return CL_OK;
}

void make_plan(const cl_layer_desc* d, Plan& p) {
  const KindInfo ki = kind_info(d->dense, d->mask);
  p.K = d->K;
  p.N = d->N;
  p.n_tiles = ceil_div(p.N, kTileRows);
  p.Npad = p.n_tiles * kTileRows;
  p.span = ki.span;
  p.chunks = ceil_div(p.K, ki.span);
  p.meta_cb = ki.meta_chunk_bytes;
  p.tab_entries = ki.table_entries;
  p.nnz = d->nnz;
  const bool has_lr = d->lr != CL_LR_NONE && d->rank > 0;
  p.rank = has_lr ? d->rank : 0;
  p.group = has_lr && d->lr == CL_LR_INT4 ? d->group : 0;

  uint64_t len[CL_SEC_COUNT] = {};
  const bool bitmap = d->mask == CL_MASK_BITMAP;
  if (bitmap) {
    p.nz_count.assign(p.N, 0);
    p.nz_off.assign(p.N + 1, 0);
    int64_t off = 0, kept = 0;
    for (int64_t n = 0; n < p.N; ++n) {
      int64_t c = 0;
      for (int64_t k = 0; k < p.K; ++k) c += d->keep[n * p.K + k] != 0;
      p.nz_count[n] = c;
      kept += c;
      p.nz_off[n] = off;
      off += round_up(c, 16);
    }
    p.nz_off[p.N] = off;
    len[CL_SEC_DENSE] = off + 64;  // slack: a lane's 16-byte loads may run past its row
    len[CL_SEC_META] = p.n_tiles * p.chunks * kTileRows * p.meta_cb;
    len[CL_SEC_NZOFF] = (p.N + 1) * 4;
    p.acct.codes = kept;
    p.acct.mask_meta = p.N * ceil_div(p.K, 32) * 4 + (p.N + 1) * 4;
  } else {
    len[CL_SEC_DENSE] = p.n_tiles * p.chunks * kTileRows * kChunkBytes;
    if (p.meta_cb) len[CL_SEC_META] = p.n_tiles * p.chunks * kTileRows * p.meta_cb;
    switch (d->dense) {
      case CL_DENSE_LUT3: p.acct.codes = p.N * ceil_div(p.K, 10) * 4; break;
      case CL_DENSE_LUT4: p.acct.codes = p.N * ceil_div(p.K, 8) * 4; break;
      case CL_DENSE_INT4:
        if (d->mask == CL_MASK_2_4) {
          p.acct.codes = p.N * (p.K / 2) / 2;     // kept values, 4 bits each
          p.acct.mask_meta = p.N * (p.K / 2) / 4; // 2 bits per kept value
        } else {
          p.acct.codes = p.N * ceil_div(p.K, 8) * 4;
        }
        break;
      case CL_DENSE_INT8: p.acct.codes = p.N * p.K; break;
    }
  }
  len[CL_SEC_TABLE] = p.tab_entries ? p.Npad * p.tab_entries * 2 : p.Npad * 2;
  p.acct.lut_or_scale = p.tab_entries ? p.N * p.tab_entries * 2 : p.N * 2;
  if (p.nnz > 0) {
    len[CL_SEC_ROWPTR] = (p.N + 1) * 4;
    len[CL_SEC_COL] = p.nnz * 4;
    len[CL_SEC_VAL] = p.nnz * 2;
    p.acct.csr = 6 * p.nnz + 4 * (p.N + 1);
  }
  if (p.rank) {
    const int64_t r = p.rank;
    if (d->lr == CL_LR_INT4) {
      p.lr_half_r = ceil_div(r, 2);
      len[CL_SEC_L] = r * ceil_div(p.K, 2);
      len[CL_SEC_R] = p.Npad * p.lr_half_r;
      len[CL_SEC_LSCALE] = ceil_div(p.K, p.group) * r * 2;
      len[CL_SEC_RSCALE] = ceil_div(r, p.group) * p.Npad * 2;
      p.acct.lowrank = ceil_div(p.K * r, 2) + 2 * ceil_div(p.K, p.group) * r + ceil_div(r * p.N, 2) +
                       2 * ceil_div(r, p.group) * p.N;
    } else {
      len[CL_SEC_L] = p.K * r * 2;
      len[CL_SEC_R] = r * p.Npad * 2;
      p.acct.lowrank = 2 * (p.K * r + r * p.N);
    }
  }
  if (d->n_xscale > 0) {
    len[CL_SEC_XSCALE] = p.K * 2;
    p.acct.act_scale = 6 * (uint64_t)d->n_xscale;
  }
  uint64_t off = round_up(sizeof(cl_blob_header), 256);
  uint64_t dev_total = 0;
  for (int s = 0; s < CL_SEC_COUNT; ++s) {
    if (!len[s]) continue;
    p.off[s] = off;
    p.len[s] = len[s];
    off = round_up(off + len[s], 256);
    dev_total += len[s];
  }
  p.total = off;
  p.acct.total = p.acct.codes + p.acct.lut_or_scale + p.acct.mask_meta + p.acct.csr + p.acct.lowrank + p.acct.act_scale;
  // every device byte of the packed sections that the canonical count does not include
  p.acct.device_padding = dev_total > p.acct.total ? dev_total - p.acct.total : 0;
}

template <class F>
void parallel_for(int64_t n, F f) {
  unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  if (n < 4 * (int64_t)nt || nt == 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::vector<std::thread> th;
  for (unsigned t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      for (int64_t i = t; i < n; i += nt) f(i);
    });
  for (auto& x : th) x.join();
}

void pack_dense(const cl_layer_desc* d, const Plan& p, uint8_t* blob) {
  const int64_t K = p.K, N = p.N, C = p.chunks;
  uint8_t* dense = blob + p.off[CL_SEC_DENSE];
  uint8_t* meta = p.len[CL_SEC_META] ? blob + p.off[CL_SEC_META] : nullptr;
  // row-major streams: chunk c of row n at (n * C + c) * chunk_bytes
  auto chunk_ptr = [&](uint8_t* base, int64_t tile, int64_t c, int64_t lane, int64_t cb) {
    return base + ((tile * kTileRows + lane) * C + c) * cb;
  };
  parallel_for(N, [&](int64_t n) {
    const int64_t tile = n / kTileRows, lane = n % kTileRows;
    if (d->dense == CL_DENSE_LUT3) {
      const uint8_t* row = d->codes + n * K;
      auto code = [&](int64_t k) -> uint32_t { return k < K ? row[k] : 0u; };
      for (int64_t c = 0; c < C; ++c) {
        uint32_t* w = reinterpret_cast<uint32_t*>(chunk_ptr(dense, tile, c, lane, 16));
        for (int i = 0; i < 4; ++i) {
          const int64_t k0 = 40 * c + 10 * i;
          uint32_t pr[5];
          for (int j = 0; j < 5; ++j) pr[j] = code(k0 + 2 * j) | (code(k0 + 2 * j + 1) << 3);
          w[i] = (pr[0] << 2) | (pr[1] << 10) | (pr[2] << 18) | (pr[3] << 26) | (pr[4] & 3u) |
                 (((pr[4] >> 2) & 3u) << 8) | (((pr[4] >> 4) & 3u) << 16);
        }
      }
    } else if (d->dense == CL_DENSE_LUT4) {
      const uint8_t* row = d->codes + n * K;
      for (int64_t c = 0; c < C; ++c) {
        uint32_t* w = reinterpret_cast<uint32_t*>(chunk_ptr(dense, tile, c, lane, 16));
        for (int i = 0; i < 4; ++i) {
          uint32_t v = 0;
          for (int b = 0; b < 4; ++b) {  // byte b: pair p = code(2b) | code(2b+1) << 4, rotated left by 2
            const int64_t k = 32 * c + 8 * i + 2 * b;
            const uint32_t pr = (k < K ? (uint32_t)row[k] : 0u) | ((k + 1 < K ? (uint32_t)row[k + 1] : 0u) << 4);
            v |= (((pr << 2) | (pr >> 6)) & 0xFFu) << (8 * b);
          }
          w[i] = v;
        }
      }
    } else if (d->dense == CL_DENSE_INT4 && d->mask == CL_MASK_NONE) {
      const int8_t* row = d->qvals + n * K;
      for (int64_t c = 0; c < C; ++c) {
        uint32_t* w = reinterpret_cast<uint32_t*>(chunk_ptr(dense, tile, c, lane, 16));
        for (int i = 0; i < 4; ++i) {
          uint32_t v = 0;
          for (int t = 0; t < 8; ++t) {
            const int64_t k = 32 * c + 8 * i + t;
            const uint32_t u = k < K ? (uint32_t)(row[k] + 8) : 8u;
            v |= u << ((t & 1) ? 16 + 4 * (t >> 1) : 4 * (t >> 1));
          }
          w[i] = v;
        }
      }
    } else if (d->dense == CL_DENSE_INT4 && d->mask == CL_MASK_2_4) {
      const int8_t* row = d->qvals + n * K;
      const uint8_t* kp = d->keep + n * K;
      for (int64_t c = 0; c < C; ++c) {
        uint32_t* w = reinterpret_cast<uint32_t*>(chunk_ptr(dense, tile, c, lane, 16));
        uint32_t* m = reinterpret_cast<uint32_t*>(chunk_ptr(meta, tile, c, lane, 8));
        for (int g = 0; g < 16; ++g) {
          const int64_t k0 = 64 * c + 4 * g;
          uint32_t i0 = 0, i1 = 1, u0 = 8, u1 = 8;
          if (k0 < K) {
            int found = 0;
            for (int t = 0; t < 4; ++t)
              if (kp[k0 + t]) (found++ == 0 ? i0 : i1) = t;
            u0 = (uint32_t)(row[k0 + i0] + 8);
            u1 = (uint32_t)(row[k0 + i1] + 8);
          }
          w[g / 4] |= (u0 << (4 * (g % 4))) | (u1 << (16 + 4 * (g % 4)));
          m[g / 8] |= (i0 | (i1 << 2)) << (4 * (g % 8));
        }
      }
    } else if (d->dense == CL_DENSE_INT8 && d->mask == CL_MASK_NONE) {
      const int8_t* row = d->qvals + n * K;
      for (int64_t c = 0; c < C; ++c) {
        uint8_t* b = chunk_ptr(dense, tile, c, lane, 16);
        for (int t = 0; t < 16; ++t) {
          const int64_t k = 16 * c + t;
          b[t] = k < K ? (uint8_t)(row[k] + 128) : 128u;
        }
      }
    } else {  // INT8 + bitmap
      const int8_t* row = d->qvals + n * K;
      const uint8_t* kp = d->keep + n * K;
      int8_t* nz = reinterpret_cast<int8_t*>(dense) + p.nz_off[n];
      int64_t j = 0;
      for (int64_t c = 0; c < C; ++c) {
        uint32_t* m = reinterpret_cast<uint32_t*>(chunk_ptr(meta, tile, c, lane, 16));
        for (int t = 0; t < 128; ++t) {
          const int64_t k = 128 * c + t;
          if (k < K && kp[k]) {
            m[t / 32] |= 1u << (t % 32);
            nz[j++] = row[k];
          }
        }
      }
    }
  });
  if (d->mask == CL_MASK_BITMAP) {
    int32_t* off = reinterpret_cast<int32_t*>(blob + p.off[CL_SEC_NZOFF]);
    for (int64_t n = 0; n <= N; ++n) off[n] = (int32_t)p.nz_off[n];
  }
}

void pack_rest(const cl_layer_desc* d, const Plan& p, uint8_t* blob) {
  const int64_t K = p.K, N = p.N;
  if (d->n_xscale > 0) {  // dense per-channel factors, fp16 1 where unscaled
    uint16_t* xs = reinterpret_cast<uint16_t*>(blob + p.off[CL_SEC_XSCALE]);
    for (int64_t k = 0; k < K; ++k) xs[k] = 0x3C00u;
    for (int32_t i = 0; i < d->n_xscale; ++i) xs[d->xscale_ch[i]] = d->xscale[i];
  }
  uint16_t* tab = reinterpret_cast<uint16_t*>(blob + p.off[CL_SEC_TABLE]);
  if (p.tab_entries)
    memcpy(tab, d->lut, N * p.tab_entries * 2);
  else
    memcpy(tab, d->row_scale, N * 2);
  if (p.nnz > 0) {
    memcpy(blob + p.off[CL_SEC_ROWPTR], d->csr_row_ptr, (N + 1) * 4);
    memcpy(blob + p.off[CL_SEC_COL], d->csr_col, p.nnz * 4);
    memcpy(blob + p.off[CL_SEC_VAL], d->csr_val, p.nnz * 2);
  }
  if (p.rank) {
    // transposed factors: L^T [r][K] and R^T [Npad][r] (see layout.h)
    const int64_t r = p.rank;
    if (d->lr == CL_LR_INT4) {
      const int8_t* L = static_cast<const int8_t*>(d->L);
      const int8_t* R = static_cast<const int8_t*>(d->R);
      const int64_t hk = ceil_div(K, 2), gk = ceil_div(K, p.group), gr = ceil_div(r, p.group);
      uint8_t* Lp = blob + p.off[CL_SEC_L];
      uint8_t* Rp = blob + p.off[CL_SEC_R];
      for (int64_t j = 0; j < r; ++j)
        for (int64_t k = 0; k < K; ++k) Lp[j * hk + k / 2] |= (uint8_t)((L[k * r + j] + 8) << (4 * (k & 1)));
      for (int64_t n = 0; n < p.Npad; ++n)
        for (int64_t j = 0; j < r; ++j) {
          const uint32_t u = n < N ? (uint32_t)(R[j * N + n] + 8) : 8u;
          Rp[n * p.lr_half_r + j / 2] |= (uint8_t)(u << (4 * (j & 1)));
        }
      uint16_t* Ls = reinterpret_cast<uint16_t*>(blob + p.off[CL_SEC_LSCALE]);
      for (int64_t g = 0; g < gk; ++g)
        for (int64_t j = 0; j < r; ++j) Ls[j * gk + g] = d->L_scale[g * r + j];
      uint16_t* Rs = reinterpret_cast<uint16_t*>(blob + p.off[CL_SEC_RSCALE]);
      for (int64_t g = 0; g < gr; ++g)
        for (int64_t n = 0; n < N; ++n) Rs[n * gr + g] = d->R_scale[g * N + n];
    } else {
      const uint16_t* L = static_cast<const uint16_t*>(d->L);
      const uint16_t* R = static_cast<const uint16_t*>(d->R);
      uint16_t* Lp = reinterpret_cast<uint16_t*>(blob + p.off[CL_SEC_L]);
      uint16_t* Rp = reinterpret_cast<uint16_t*>(blob + p.off[CL_SEC_R]);
      for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < r; ++j) Lp[j * K + k] = L[k * r + j];
      for (int64_t j = 0; j < r; ++j)
        for (int64_t n = 0; n < N; ++n) Rp[n * r + j] = R[j * N + n];
    }
  }
}

}  // namespace
}  // namespace cl

using namespace cl;

extern "C" cl_status cl_pack(const cl_layer_desc* d, void* blob, size_t* blob_bytes, cl_bytes* acct) {
  clear_error();
  if (!blob_bytes) return fail(CL_EINVAL, "blob_bytes is NULL");
  cl_status st = validate(d);
  if (st != CL_OK) return st;
  Plan p;
  make_plan(d, p);
  for (int sct = 0; sct < CL_SEC_COUNT; ++sct)
    if (p.len[sct] >= kMaxBufferBytes)
      return fail(CL_ESIZE, "section %d of the device layout would hold %llu bytes (at most 2^31 - 1)", sct,
                  (unsigned long long)p.len[sct]);
  if (acct) *acct = p.acct;
  if (!blob) {
    *blob_bytes = p.total;
    return CL_OK;
  }
  if (reinterpret_cast<uintptr_t>(blob) % 16) return fail(CL_EINVAL, "blob must be 16-byte aligned");
  if (*blob_bytes < p.total) {
    const size_t cap = *blob_bytes;
    *blob_bytes = p.total;
    return fail(CL_ENOMEM, "blob needs %zu bytes, got %zu", (size_t)p.total, cap);
  }
  uint8_t* b = static_cast<uint8_t*>(blob);
  memset(b, 0, p.total);
  cl_blob_header* h = reinterpret_cast<cl_blob_header*>(b);
  h->magic = CL_BLOB_MAGIC;
  h->version = CL_BLOB_VERSION;
  h->K = d->K;
  h->N = d->N;
  h->dense = d->dense;
  h->mask = d->mask;
  h->lr = p.rank ? d->lr : CL_LR_NONE;
  h->rank = (int32_t)p.rank;
  h->group = (int32_t)p.group;
  h->x_dtype = d->x_dtype;
  h->has_clamp = d->has_clamp ? 1 : 0;
  h->act_clamp = d->has_clamp ? d->act_clamp : 0;
  h->n_tiles = (int32_t)p.n_tiles;
  h->chunks = (int32_t)p.chunks;
  h->span = (int32_t)p.span;
  h->meta_chunk_bytes = (int32_t)p.meta_cb;
  h->nnz = p.nnz;
  h->total_bytes = p.total;
  for (int s = 0; s < CL_SEC_COUNT; ++s) {
    h->off[s] = p.off[s];
    h->len[s] = p.len[s];
  }
  h->acct = p.acct;
  h->n_xscale = d->n_xscale;
  pack_dense(d, p, b);
  pack_rest(d, p, b);
  *blob_bytes = p.total;
  return CL_OK;
}

extern "C" const char* cl_last_error(void) { return g_err.c_str(); }
