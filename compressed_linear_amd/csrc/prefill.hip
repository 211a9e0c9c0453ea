// prefill.hip -- large-M forward: dispatch of the MFMA kernels.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "layer.h"
#include "prefill_impl.h"

namespace cl {

extern template hipError_t launch_prefill_kind<K_LUT3>(const PfArgs&, bool, hipStream_t);
extern template hipError_t launch_prefill_kind<K_LUT4>(const PfArgs&, bool, hipStream_t);
extern template hipError_t launch_prefill_kind<K_INT4>(const PfArgs&, bool, hipStream_t);
extern template hipError_t launch_prefill_kind<K_INT4_24>(const PfArgs&, bool, hipStream_t);
extern template hipError_t launch_prefill_kind<K_INT8>(const PfArgs&, bool, hipStream_t);
extern template hipError_t launch_prefill_kind<K_DENSE16>(const PfArgs&, bool, hipStream_t);
extern template hipError_t launch_prefill_kind<K_DENSE_INT4>(const PfArgs&, bool, hipStream_t);

// The bitmap format has no matrix-core loader yet: row blocks of 32 through the decode kernels.
static hipError_t prefill_by_decode(const Layer& L, int M, const void* x, float* y, hipStream_t stream) {
  const int ldx = (x == L.xprep) ? L.Kx : L.h.K;
  for (int m0 = 0; m0 < M; m0 += kMaxDecodeM) {
    const int mb = M - m0 < kMaxDecodeM ? M - m0 : kMaxDecodeM;
    const void* xb = static_cast<const uint16_t*>(x) + (size_t)m0 * ldx;
    Layer Lb = L;
    if (x == L.xprep) Lb.xprep = const_cast<uint16_t*>(static_cast<const uint16_t*>(xb));
    hipError_t e = hipSuccess;
    if (L.h.lr != CL_LR_NONE) e = launch_lowrank_prologue(Lb, mb, xb, stream);
    if (e == hipSuccess) e = launch_decode(Lb, mb, xb, y + (size_t)m0 * L.h.N, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int KIND>
static int dense_steps(const cl_blob_header& h) {
  return (int)ceil_div(h.chunks, PfCfg<KIND>::bk / PfCfg<KIND>::span);
}

hipError_t launch_prefill(const Layer& L, int M, const void* x, float* y, hipStream_t stream) {
  const cl_blob_header& h = L.h;
  if (h.mask == CL_MASK_BITMAP) return prefill_by_decode(L, M, x, y, stream);
  const bool bf16 = h.x_dtype == CL_ACT_BF16;
  PfArgs a = {};
  a.x = static_cast<const uint16_t*>(x);
  a.ldx = (x == L.xprep) ? L.Kx : h.K;
  a.M = M;
  a.K = h.K;
  const bool has_lr = h.lr != CL_LR_NONE && h.rank > 0;
  const int rp = (int)round_up(h.rank, 8);
  hipError_t e = hipSuccess;
  if (has_lr) {
    // t = x' L on the matrix cores: L^T rows are the weight tile; t is [M][rp], zero past the rank
    PfArgs p = a;
    p.N = h.rank;
    p.Npad = h.rank;
    p.group = h.group > 0 ? h.group : 1;
    p.b_bf16 = h.lr == CL_LR_BF16;
    p.y = L.t;
    p.ldy = rp;
    p.ncols = rp;
    p.nsteps = p.nsteps_dense = (int)ceil_div(h.K, PfCfg<K_DENSE16>::bk);
    if (h.lr == CL_LR_INT4) {
      p.b4 = L.L;
      p.b4s = L.Lscale;
      e = launch_prefill_kind<K_DENSE_INT4>(p, bf16, stream);
    } else {
      p.b16 = reinterpret_cast<const uint16_t*>(L.L);
      e = launch_prefill_kind<K_DENSE16>(p, bf16, stream);
    }
    if (e != hipSuccess) return e;
  }
  a.N = h.N;
  a.Npad = L.Npad;
  a.dense = reinterpret_cast<const uint4*>(L.dense);
  a.meta = L.meta;
  a.table = reinterpret_cast<const uint16_t*>(L.table);
  a.chunks = h.chunks;
  if (h.nnz > 0) {
    a.rowptr = L.rowptr;
    a.col = L.col;
    a.val = L.val;
  }
  if (has_lr) {
    a.t = L.t;
    a.ldt = rp;
    a.rank = h.rank;
    a.rp = rp;
    a.lr_kind = h.lr;
    a.R = L.R;
    a.Rscale = L.Rscale;
    a.rgroup = h.group > 0 ? h.group : 1;
  }
  a.y = y;
  a.ldy = h.N;
  a.ncols = h.N;
  auto run = [&](auto kind_tag, int bk) {
    constexpr int KIND = decltype(kind_tag)::value;
    a.nsteps_dense = dense_steps<KIND>(h);
    a.nsteps = a.nsteps_dense + (has_lr ? (int)ceil_div(2 * rp, bk) : 0);
    return launch_prefill_kind<KIND>(a, bf16, stream);
  };
  switch (h.dense) {
    case CL_DENSE_LUT3: return run(std::integral_constant<int, K_LUT3>{}, PfCfg<K_LUT3>::bk);
    case CL_DENSE_LUT4: return run(std::integral_constant<int, K_LUT4>{}, PfCfg<K_LUT4>::bk);
    case CL_DENSE_INT4:
      return h.mask == CL_MASK_2_4 ? run(std::integral_constant<int, K_INT4_24>{}, PfCfg<K_INT4_24>::bk)
                                   : run(std::integral_constant<int, K_INT4>{}, PfCfg<K_INT4>::bk);
    default: return run(std::integral_constant<int, K_INT8>{}, PfCfg<K_INT8>::bk);
  }
}

}  // namespace cl
