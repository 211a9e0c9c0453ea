// decode.hip -- dispatch of the batch 1..32 forward: the row-wise kernel for
// M <= 3 (M = 1 with bf16 activations) when its staged activations fit in LDS, the matrix-core decode kernel
// for larger batches and the row-wise kernel's misfits, the tile kernel for the
// bitmap format (and for layers created for batch 1 only).
#include "decode_impl.h"
#include "decode_mfma.h"
#include "decode_rows.h"
#include "decode_stream.h"

#include <algorithm>

namespace cl {

extern template hipError_t launch_decode_kind<K_LUT3>(const DecodeArgs&, bool, hipStream_t);
extern template hipError_t launch_decode_kind<K_LUT4>(const DecodeArgs&, bool, hipStream_t);
extern template hipError_t launch_decode_kind<K_INT4>(const DecodeArgs&, bool, hipStream_t);
extern template hipError_t launch_decode_kind<K_INT4_24>(const DecodeArgs&, bool, hipStream_t);
extern template hipError_t launch_decode_kind<K_INT8>(const DecodeArgs&, bool, hipStream_t);
extern template hipError_t launch_decode_kind<K_INT8_BM>(const DecodeArgs&, bool, hipStream_t);

extern template hipError_t launch_rows_kind<K_LUT3>(const RowArgs&, int, bool, hipStream_t);
extern template hipError_t launch_rows_kind<K_LUT4>(const RowArgs&, int, bool, hipStream_t);
extern template hipError_t launch_rows_kind<K_INT4>(const RowArgs&, int, bool, hipStream_t);
extern template hipError_t launch_rows_kind<K_INT4_24>(const RowArgs&, int, bool, hipStream_t);
extern template hipError_t launch_rows_kind<K_INT8>(const RowArgs&, int, bool, hipStream_t);

extern template hipError_t launch_stream_kind<K_LUT3>(const StreamArgs&, int, int, int, bool, hipStream_t);
extern template hipError_t launch_stream_kind<K_LUT4>(const StreamArgs&, int, int, int, bool, hipStream_t);
extern template hipError_t launch_stream_kind<K_INT4>(const StreamArgs&, int, int, int, bool, hipStream_t);
extern template hipError_t launch_stream_kind<K_INT4_24>(const StreamArgs&, int, int, int, bool, hipStream_t);
extern template hipError_t launch_stream_kind<K_INT8>(const StreamArgs&, int, int, int, bool, hipStream_t);

extern template hipError_t launch_mfma_kind<K_LUT3>(const MfArgs&, bool, hipStream_t);
extern template hipError_t launch_mfma_kind<K_LUT4>(const MfArgs&, bool, hipStream_t);
extern template hipError_t launch_mfma_kind<K_INT4>(const MfArgs&, bool, hipStream_t);
extern template hipError_t launch_mfma_kind<K_INT4_24>(const MfArgs&, bool, hipStream_t);
extern template hipError_t launch_mfma_kind<K_INT8>(const MfArgs&, bool, hipStream_t);
extern template hipError_t launch_mfma_kind<K_INT8_BM>(const MfArgs&, bool, hipStream_t);

// Smallest batch that the automatic choice sends to the matrix-core decode kernel.
constexpr int kMfMinM = 4;

// The epoch a launch with the low-rank prologue inside publishes: a new nonzero
// value per direct call; 0 while the stream is being recorded into a graph (the
// launch then derives its generation on the device, so replays stay valid).
static uint32_t next_epoch(const Layer& L, hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) == hipSuccess && st != hipStreamCaptureStatusNone) return 0u;
  if (++L.lr_epoch == 0) ++L.lr_epoch;
  return L.lr_epoch;
}

// Whether the decode kernels can read the caller's activations raw and edit
// them (the clamp, the per-channel factors) while staging them: rows of
// 16-byte aligned loads (K a multiple of 8) and no low-rank prologue kernel of
// its own (that kernel reads edited activations).
static bool edit_in_kernel(const Layer& L) {
  return L.h.K % 8 == 0 && (L.h.lr == CL_LR_NONE || L.lr_mode >= 0);
}

// x: the caller's activations, or L.xprep when they are edited / restaged
// already.  The matrix-core kernel reads them raw where edit_in_kernel allows
// (the low-rank prologue, if any, then runs inside the same launch and edits
// them the same way); otherwise a prep kernel runs first.
static hipError_t launch_decode_mfma(const Layer& L, int M, const void* x, float* y, hipStream_t stream) {
  const cl_blob_header& h = L.h;
  const bool has_lr = h.lr != CL_LR_NONE;
  const bool fused_lr = has_lr && L.lr_mode >= 0;
  const bool raw = L.xprep != nullptr && x != L.xprep;
  bool edit = false;
  if (raw) {
    if (edit_in_kernel(L)) {
      edit = true;
    } else {
      const hipError_t e = launch_prep_x(L, M, x, stream);
      if (e != hipSuccess) return e;
      x = L.xprep;
    }
  }
  if (has_lr && !fused_lr) {
    const hipError_t e = launch_lowrank_prologue(L, M, x, stream);
    if (e != hipSuccess) return e;
  }
  MfArgs a = {};
  a.dense = reinterpret_cast<const uint4*>(L.dense);
  a.meta = L.meta;
  a.table = reinterpret_cast<const uint16_t*>(L.table);
  a.x = x;
  a.ldx = (x == L.xprep) ? L.Kx : h.K;
  a.M = M;
  a.K = h.K;
  a.N = h.N;
  a.Npad = L.Npad;
  a.chunks = h.chunks;
  a.tiles = L.mf_tiles;
  a.S = L.mf_S;
  a.Kz = L.mf_Kz;
  a.npw = L.mf_npw;
  a.ooff = h.nnz > 0 ? L.mf_ooff : nullptr;
  a.oent = L.mf_oent;
  a.nnz = (int)h.nnz;
  a.nzs = L.mf_nzs;
  a.dense_bytes = (uint32_t)h.len[CL_SEC_DENSE];
  a.r16 = h.lr != CL_LR_NONE ? L.pf_r16 : nullptr;
  a.t = L.t;
  a.rank = h.rank;
  a.rp = L.pf_rp;
  a.part = L.mf_part;
  a.counters = L.counters;
  a.y = y;
  a.clamp = edit && h.has_clamp ? 1 : 0;
  a.cval = (float)__builtin_bit_cast(_Float16, h.act_clamp);
  a.xscale = edit ? L.xscale : nullptr;
  if (fused_lr) {
    a.lrp = lowrank_split_args(L, M, x);
    a.lr_ntj = L.lr_rpad / 64;
    a.lrp.ntiles = a.lr_ntj * (int)ceil_div(M, kMfLrTile);
    a.lrp.flag = L.lr_cnt + 65;
    a.lrp.epoch = next_epoch(L, stream);
    a.lrp.clamp = a.clamp;
    a.lrp.cval = a.cval;
    a.lrp.xscale = a.xscale;
    a.lrp.withhold = L.wait_withhold;
    a.lr_wgs = L.lr_S * a.lrp.ntiles;
    a.lr_mode = L.lr_mode;
    a.lr_max_polls = L.wait_polls;
    a.lr_err = L.wait_err_dev;
  }
  const bool bf16 = h.x_dtype == CL_ACT_BF16;
  switch (h.dense) {
    case CL_DENSE_LUT3: return launch_mfma_kind<K_LUT3>(a, bf16, stream);
    case CL_DENSE_LUT4: return launch_mfma_kind<K_LUT4>(a, bf16, stream);
    case CL_DENSE_INT4:
      return h.mask == CL_MASK_2_4 ? launch_mfma_kind<K_INT4_24>(a, bf16, stream) : launch_mfma_kind<K_INT4>(a, bf16, stream);
    default:
      return h.mask == CL_MASK_BITMAP ? launch_mfma_kind<K_INT8_BM>(a, bf16, stream) : launch_mfma_kind<K_INT8>(a, bf16, stream);
  }
}

// ---------------------------------------------------------------------------
// Batch 1 on the streaming kernel: the plan (rows per workgroup, wavefronts per
// workgroup, LDS layout) is made at create so that every workgroup is resident
// at once: one workgroup of 16 wavefronts per CU, or two of 8 when the LDS of
// one does not allow 16.
// ---------------------------------------------------------------------------
static size_t a16(size_t v) { return (v + 15) & ~(size_t)15; }

template <int KIND>
static StreamPlanH plan_stream_k(const cl_blob_header& h, const int32_t* rp, int num_cus, int lr_mode) {
  StreamPlanH p;
  constexpr bool LUT = KIND == K_LUT3 || KIND == K_LUT4;
  constexpr int RTB = row_table_bytes<KIND>();
  constexpr int TB = KIND == K_LUT4 ? 32 : KIND == K_LUT3 ? 16 : 2;
  const int N = h.N, C = (int)h.chunks;
  // outlier columns are packed in 16 bits; a pass meets at most one row boundary
  if (h.K > 65535 || C < 64) return p;
  const bool lr = h.lr != CL_LR_NONE && h.rank > 0, lr4 = h.lr == CL_LR_INT4;
  if (lr && h.rank > 256) return p;
  const int rrb = lr ? (lr4 ? (h.rank + 1) / 2 : 2 * h.rank) : 0;
  const int rscb = lr4 ? 2 * (int)ceil_div(h.rank, h.group) : 0;
  if (lr && (rrb % 2 || rscb % 2)) return p;
  // rank rows and scales are staged with 16-byte loads: rows per workgroup a multiple of m
  int m = 1;
  while ((m * rrb) % 16 || (m * rscb) % 16) m *= 2;
  for (int wpg = kStMaxWaves; wpg >= 8; wpg /= 2) {
    const int threads = wpg * 64, k = kStMaxWaves / wpg;  // workgroups per CU
    if (stream_slots_per_thread<KIND>(C, threads) > 12) continue;
    // the prologue workgroups (the launch's first) hold their CUs while they
    // run: the row workgroups take the others, so that none waits for a CU
    // int4 factors in 1024-thread blocks: 512-row slices while that needs at
    // most 16 blocks, else 2048-row ones (fewer CUs taken from the rows; their
    // longer dequantisation still ends before the walk).  Measured, SLiM int4
    // rank 128, us per layer with 512 / 1024 / 2048-row slices: 4096 -> 11008
    // 10.5 / 10.9 / 13.4, 11008 -> 4096 14.1 / 13.9 / 13.6.
    const int lr_S = (int)ceil_div(h.K, kLrSlice), ntj = (int)ceil_div(h.rank, 64);
    const int nl = (lr && lr_mode == 1 && threads == 1024 && stream_lr_slices(lr_S, threads, 1, 1) * ntj > 16) ? 4 : 1;
    const int lr_wgs = (lr && lr_mode >= 0) ? stream_lr_slices(lr_S, threads, lr_mode, nl) * ntj : 0;
    const size_t lr_lds = lr_wgs ? (size_t)lr_scratch_bytes(lr_mode, 1, threads == 1024 ? 1024 : 256, nl) : 0;
    const long long slots = (long long)num_cus * k - lr_wgs;
    if (slots < (long long)num_cus * k / 2) continue;
    const int RW = (int)(ceil_div(ceil_div(N, slots), m) * m);
    if (RW + 1 > threads) continue;                       // one row (pointer) per thread
    if (LUT && RW * RTB > stream_tab_bytes<KIND>()) continue;  // row tables in the static array
    if ((long long)RW * rrb > 2LL * 16 * threads || (long long)RW * rscb > 16LL * threads) continue;
    const int nwg = (int)ceil_div(N, RW);
    long long most = 0;  // outliers of the busiest workgroup
    if (rp)
      for (int w = 0; w < nwg; ++w) {
        const int r0 = w * RW, r1 = r0 + RW < N ? r0 + RW : N;
        most = std::max<long long>(most, (long long)rp[r1] - rp[r0]);
      }
    const int cap = (int)std::min<long long>(most, (long long)kStOutLoads * threads);
    StreamPlanH t;
    size_t off = 0;
    t.lds_x = (int)off;
    off += a16((size_t)C * RowX<KIND>::stride);
    t.lds_max = (int)off;
    off += (size_t)kStMaxWaves * 4;
    t.lds_meta = (int)off;
    off += a16((size_t)RW * TB);
    t.lds_rp = (int)off;
    off += a16((size_t)(RW + 1) * 4);
    const int rrs = rrb >= 16 && (rrb & (rrb - 1)) == 0 ? rrb + 16 : rrb;  // padded: rows read together on other banks
    t.lds_rank = (int)off;
    off += a16((size_t)RW * rrs);
    t.lds_rsc = (int)off;
    off += a16((size_t)RW * rscb);
    t.lds_part0 = (int)off;
    off += (size_t)RW * 256;
    t.lds_part1 = (int)off;
    off += (size_t)wpg * 256;
    t.lds_out = (int)off;
    off += a16((size_t)cap * 4);  // columns and values, 16 bits each
    t.lds_t = (int)off;
    off += lr ? (size_t)h.rank * 4 : 0;
    const size_t dyn = off > lr_lds ? off : lr_lds;
    if ((size_t)k * (dyn + stream_tab_bytes<KIND>()) > 160 * 1024) continue;
    t.ok = 1;
    t.wpg = wpg;
    t.rows_per_wg = RW;
    t.nwg = nwg;
    t.lds = (int)dyn;
    t.out_cap = cap;
    t.rank_row_bytes = rrb;
    t.lr_nl = nl;
    t.rank_row_stride = rrs;
    t.rsc_row_bytes = rscb;
    return t;
  }
  return p;
}

// Which batch-1 layers take the streaming kernel.  Its launch costs a fixed
// few microseconds (dispatch of full-CU workgroups, staging the activations and
// row tables once per CU) and then streams at close to the memory rate; the
// row-wise kernel starts at once but streams slower.  With a rank term, the
// streaming kernel's prologue hands t to its readers in one trip through memory
// (tagged partial sums), the row-wise kernel's in several.  Measured on one
// MI355X (us per layer, streaming / row-wise): LLaMA-70B LUT3 + bf16 rank 64
// 8192 -> 10240 (32 MiB of codes) 16.1 / 16.6, 8192 -> 28672 29.5 / 37.9,
// 28672 -> 8192 30.4 / 36.9; INT4 2:4 + int4 rank 128 4096 -> 11008 (11 MiB)
// 10.5 / 15.3, 11008 -> 4096 14.2 / 14.9; LLaMA-7B LUT4 4096 -> 12288 (24 MiB)
// 12.5 / 9.8; LUT3 4096 -> 4096 7.3 / 4.9.  The streaming kernel takes layers
// of 28 MiB of codes or more, and layers with a rank term.
static bool stream_wins(const cl_blob_header& h) {
  const bool lr = h.lr != CL_LR_NONE && h.rank > 0;
  return (unsigned long long)h.N * h.chunks * 16ull >= (28ull << 20) || lr;
}

StreamPlanH plan_stream(const cl_blob_header& h, const int32_t* rowptr, int num_cus, int lr_mode) {
  const int32_t* rp = h.nnz > 0 ? rowptr : nullptr;
  StreamPlanH p;
  switch (h.dense) {
    case CL_DENSE_LUT3: p = plan_stream_k<K_LUT3>(h, rp, num_cus, lr_mode); break;
    case CL_DENSE_LUT4: p = plan_stream_k<K_LUT4>(h, rp, num_cus, lr_mode); break;
    case CL_DENSE_INT4:
      p = h.mask == CL_MASK_2_4 ? plan_stream_k<K_INT4_24>(h, rp, num_cus, lr_mode)
                                : plan_stream_k<K_INT4>(h, rp, num_cus, lr_mode);
      break;
    default:
      if (h.mask == CL_MASK_BITMAP) return StreamPlanH();
      p = plan_stream_k<K_INT8>(h, rp, num_cus, lr_mode);
  }
  p.pick = p.ok && stream_wins(h);
  return p;
}

static hipError_t launch_decode_stream(const Layer& L, const void* x, float* y, hipStream_t stream) {
  const cl_blob_header& h = L.h;
  const bool bf16 = h.x_dtype == CL_ACT_BF16;
  const bool raw = L.xprep != nullptr && x != L.xprep;
  bool edit = false;
  if (raw) {
    if (edit_in_kernel(L)) {
      edit = true;
    } else {
      const hipError_t e = launch_prep_x(L, 1, x, stream);
      if (e != hipSuccess) return e;
      x = L.xprep;
    }
  }
  StreamArgs s = {};
  RowArgs& r = s.r;
  r.dense = reinterpret_cast<const uint4*>(L.dense);
  r.meta = L.meta;
  r.table = reinterpret_cast<const uint16_t*>(L.table);
  r.rowptr = h.nnz > 0 ? L.rowptr : nullptr;
  r.col = L.col;
  r.val = L.val;
  r.R = L.R;
  r.Rscale = L.Rscale;
  r.t = L.t;
  r.x = x;
  r.ldx = (x == L.xprep) ? L.Kx : h.K;
  r.y = y;
  r.K = h.K;
  r.N = h.N;
  r.M = 1;
  r.chunks = h.chunks;
  r.rank = h.lr != CL_LR_NONE ? h.rank : 0;
  r.group = h.group > 0 ? h.group : 1;
  r.group_mul = (uint32_t)((65536 + r.group - 1) / r.group);
  r.lr_kind = h.lr;
  r.Npad = L.Npad;
  r.nnz = (int)h.nnz;
  r.clamp = edit && h.has_clamp ? 1 : 0;
  r.cval = (float)__builtin_bit_cast(_Float16, h.act_clamp);
  r.xscale = edit ? L.xscale : nullptr;
  int lr_lds = 0;
  if (h.lr != CL_LR_NONE) {
    if (L.lr_mode >= 0) {  // the prologue runs as this launch's first workgroups
      r.lrp = lowrank_split_args(L, 1, x);
      r.lrp.clamp = r.clamp;
      r.lrp.cval = r.cval;
      r.lrp.xscale = r.xscale;
      r.lrp.flag = L.lr_cnt + 65;
      r.lrp.epoch = next_epoch(L, stream);
      r.lrp.withhold = L.wait_withhold;
      r.lrp.S = stream_lr_slices(L.lr_S, L.st.wpg * 64, L.lr_mode, L.st.lr_nl);  // blocks over longer K slices
      r.lr_ntj = L.lr_rpad / 64;
      r.lr_wgs = r.lrp.S * r.lr_ntj;
      r.lr_mode = L.lr_mode;
      r.lr_flag = r.lrp.flag;
      r.lr_epoch = r.lrp.epoch;
      r.lr_max_polls = L.wait_polls;
      r.lr_err = L.wait_err_dev;
      lr_lds = lr_scratch_bytes(L.lr_mode, 1, L.st.wpg * 64 == 1024 ? 1024 : 256, L.st.lr_nl);
    } else {
      const hipError_t e = launch_lowrank_prologue(L, 1, x, stream);
      if (e != hipSuccess) return e;
    }
  }
  const StreamPlanH& p = L.st;
  s.rows_per_wg = p.rows_per_wg;
  s.lds_x = p.lds_x;
  s.lds_max = p.lds_max;
  s.lds_meta = p.lds_meta;
  s.lds_rp = p.lds_rp;
  s.lds_rank = p.lds_rank;
  s.lds_rsc = p.lds_rsc;
  s.lds_part0 = p.lds_part0;
  s.lds_part1 = p.lds_part1;
  s.lds_out = p.lds_out;
  s.lds_t = p.lds_t;
  s.rank_row_bytes = p.rank_row_bytes;
  s.rank_row_stride = p.rank_row_stride;
  s.rsc_row_bytes = p.rsc_row_bytes;
  s.out_cap = p.out_cap;
  s.lr_readers = p.nwg;
  s.lr_nl = p.lr_nl;
  const int lds = p.lds > lr_lds ? p.lds : lr_lds;
  const int grid = r.lr_wgs + p.nwg, threads = p.wpg * 64;
  switch (h.dense) {
    case CL_DENSE_LUT3: return launch_stream_kind<K_LUT3>(s, grid, threads, lds, bf16, stream);
    case CL_DENSE_LUT4: return launch_stream_kind<K_LUT4>(s, grid, threads, lds, bf16, stream);
    case CL_DENSE_INT4:
      return h.mask == CL_MASK_2_4 ? launch_stream_kind<K_INT4_24>(s, grid, threads, lds, bf16, stream)
                                   : launch_stream_kind<K_INT4>(s, grid, threads, lds, bf16, stream);
    default: return launch_stream_kind<K_INT8>(s, grid, threads, lds, bf16, stream);
  }
}

hipError_t launch_decode(const Layer& L, int M, const void* x, float* y, hipStream_t stream, int variant) {
  // batch 1: the streaming kernel where it is the faster one for the layer's shape
  if (M == 1 && L.st.ok && (variant == 3 || (variant == 0 && L.st.pick))) return launch_decode_stream(L, x, y, stream);

  // bf16 activations cost the row-wise kernel two multiply-adds per weight pair
  // and activation row (no mixed fp16 x bf16 dot product), so it keeps only batch 1
  const bool mf_auto = M >= kMfMinM || (M >= 2 && L.h.x_dtype == CL_ACT_BF16);
  if (L.mf_S > 0 && (variant == 2 || (variant == 0 && mf_auto))) return launch_decode_mfma(L, M, x, y, stream);

  const cl_blob_header& h = L.h;
  const bool bf16 = h.x_dtype == CL_ACT_BF16;
  const bool raw = L.xprep != nullptr && x != L.xprep;
  // M <= 4: row-wise kernel (bandwidth bound) when its staged activations fit
  // in LDS; the bitmap format always uses the tile kernel (its kept values are
  // consumed per row at a varying rate).  The row-wise kernel edits raw
  // activations while staging them where edit_in_kernel allows and its first
  // staging round holds the whole activation block; the tile kernel reads
  // edited / restaged ones.
  RowArgs r = {};
  bool rows = false, rows_edit = false;
  if (M <= 4 && h.mask != CL_MASK_BITMAP) {
    r.dense = reinterpret_cast<const uint4*>(L.dense);
    r.meta = L.meta;
    r.table = reinterpret_cast<const uint16_t*>(L.table);
    r.rowptr = h.nnz > 0 ? L.rowptr : nullptr;
    r.col = L.col;
    r.val = L.val;
    r.R = L.R;
    r.Rscale = L.Rscale;
    r.t = L.t;
    r.y = y;
    r.K = h.K;
    r.N = h.N;
    r.M = M;
    r.chunks = h.chunks;
    r.rank = h.lr != CL_LR_NONE ? h.rank : 0;
    r.group = h.group > 0 ? h.group : 1;
    r.group_mul = (uint32_t)((65536 + r.group - 1) / r.group);
    r.lr_kind = h.lr;
    r.Npad = L.Npad;
    r.nnz = (int)h.nnz;
    bool one_round = false;
    switch (h.dense) {
      case CL_DENSE_LUT3: rows = rows_fit<K_LUT3>(r, bf16, &one_round); break;
      case CL_DENSE_LUT4: rows = rows_fit<K_LUT4>(r, bf16, &one_round); break;
      case CL_DENSE_INT4:
        rows = h.mask == CL_MASK_2_4 ? rows_fit<K_INT4_24>(r, bf16, &one_round) : rows_fit<K_INT4>(r, bf16, &one_round);
        break;
      default: rows = rows_fit<K_INT8>(r, bf16, &one_round); break;
    }
    rows_edit = rows && raw && one_round && edit_in_kernel(L);
  }
  // batches the row-wise kernel cannot stage: the matrix-core kernel where it applies
  if (!rows && variant == 0 && L.mf_S > 0) return launch_decode_mfma(L, M, x, y, stream);
  if (raw && !rows_edit) {
    const hipError_t e = launch_prep_x(L, M, x, stream);
    if (e != hipSuccess) return e;
    x = L.xprep;
  }
  const int ldx = (x == L.xprep) ? L.Kx : h.K;

  if (rows) {
    r.x = x;
    r.ldx = ldx;
    r.clamp = rows_edit && h.has_clamp ? 1 : 0;
    r.cval = (float)__builtin_bit_cast(_Float16, h.act_clamp);
    r.xscale = rows_edit ? L.xscale : nullptr;
    if (h.lr != CL_LR_NONE) {
      if (L.lr_mode >= 0) {
        // the prologue runs as this launch's first workgroups
        r.lrp = lowrank_split_args(L, M, x);
        r.lrp.clamp = r.clamp;
        r.lrp.cval = r.cval;
        r.lrp.xscale = r.xscale;
        r.lrp.flag = L.lr_cnt + 65;
        r.lrp.epoch = next_epoch(L, stream);
        r.lr_ntj = L.lr_rpad / 64;
        r.lr_wgs = L.lr_S * r.lr_ntj * (int)ceil_div(M, lowrank_tile_m(M));
        r.lr_mode = L.lr_mode;
        r.lrp.withhold = L.wait_withhold;
        r.lr_flag = r.lrp.flag;
        r.lr_epoch = r.lrp.epoch;
        r.lr_max_polls = L.wait_polls;
        r.lr_err = L.wait_err_dev;
      } else {
        const hipError_t e = launch_lowrank_prologue(L, M, x, stream);
        if (e != hipSuccess) return e;
      }
    }
    switch (h.dense) {
      case CL_DENSE_LUT3: return launch_rows_kind<K_LUT3>(r, L.Npad, bf16, stream);
      case CL_DENSE_LUT4: return launch_rows_kind<K_LUT4>(r, L.Npad, bf16, stream);
      case CL_DENSE_INT4:
        return h.mask == CL_MASK_2_4 ? launch_rows_kind<K_INT4_24>(r, L.Npad, bf16, stream)
                                     : launch_rows_kind<K_INT4>(r, L.Npad, bf16, stream);
      default: return launch_rows_kind<K_INT8>(r, L.Npad, bf16, stream);
    }
  }

  DecodeArgs a = {};
  a.dense = reinterpret_cast<const uint4*>(L.dense);
  a.meta = L.meta;
  a.nzstart = L.nzstart;
  a.table = reinterpret_cast<const uint16_t*>(L.table);
  a.rowptr = h.nnz > 0 ? L.rowptr : nullptr;
  a.col = L.col;
  a.val = L.val;
  a.R = L.R;
  a.Rscale = L.Rscale;
  a.t = L.t;
  a.x = x;
  a.y = y;
  a.part = L.part;
  a.counters = L.counters;
  a.K = h.K;
  a.N = h.N;
  a.M = M;
  a.ldx = ldx;
  a.chunks = h.chunks;
  a.span = h.span;
  a.split = L.split;
  a.G = h.n_tiles * L.split;
  a.Gpad = (a.G + 7) & ~7;
  a.rank = h.rank;
  a.group = h.group > 0 ? h.group : 1;
  a.lr_kind = h.lr;
  a.Npad = L.Npad;
  if (h.lr != CL_LR_NONE) {
    const hipError_t e = launch_lowrank_prologue(L, M, x, stream);
    if (e != hipSuccess) return e;
  }
  switch (h.dense) {
    case CL_DENSE_LUT3: return launch_decode_kind<K_LUT3>(a, bf16, stream);
    case CL_DENSE_LUT4: return launch_decode_kind<K_LUT4>(a, bf16, stream);
    case CL_DENSE_INT4:
      return h.mask == CL_MASK_2_4 ? launch_decode_kind<K_INT4_24>(a, bf16, stream) : launch_decode_kind<K_INT4>(a, bf16, stream);
    default:
      return h.mask == CL_MASK_BITMAP ? launch_decode_kind<K_INT8_BM>(a, bf16, stream) : launch_decode_kind<K_INT8>(a, bf16, stream);
  }
}

}  // namespace cl
