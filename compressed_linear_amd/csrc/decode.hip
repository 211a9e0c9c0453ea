// decode.hip -- dispatch of the batch 1..32 forward: the row-wise kernel for
// M <= 3 (M = 1 with bf16 activations) when its staged activations fit in LDS, the matrix-core decode kernel
// for larger batches and the row-wise kernel's misfits, the tile kernel for the
// bitmap format (and for layers created for batch 1 only).
#include "decode_impl.h"
#include "decode_mfma.h"
#include "decode_rows.h"

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

hipError_t launch_decode(const Layer& L, int M, const void* x, float* y, hipStream_t stream, int variant) {
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
