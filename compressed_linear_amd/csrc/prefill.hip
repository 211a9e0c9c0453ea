// prefill.hip -- large-M forward: dispatch of the MFMA kernels.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "layer.h"
#include "prefill_impl.h"

namespace cl {

extern template hipError_t launch_prefill_kind<K_LUT4>(const PfArgs&, bool, hipStream_t);
extern template hipError_t launch_prefill_kind<K_INT4>(const PfArgs&, bool, hipStream_t);
extern template hipError_t launch_prefill_kind<K_INT4_24>(const PfArgs&, bool, hipStream_t);
extern template hipError_t launch_prefill_kind<K_INT8>(const PfArgs&, bool, hipStream_t);
extern template hipError_t launch_prefill_kind<K_DENSE16>(const PfArgs&, bool, hipStream_t);
hipError_t launch_prefill_wide(const PfArgs& a, bool bf16, hipStream_t stream);  // the 3-bit LUT format

// t_hi | t_lo of t = the sum of the prologue's K-split partials, added in a
// fixed order: [M][2 rp], t_hi = t rounded to the MFMA type, t_lo = the rest.
template <bool BF16>
__global__ void __launch_bounds__(256) pf_tsplit_kernel(const float* t, size_t tstride, int split, int M, int rp,
                                                        uint16_t* t16) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * 2 * rp) return;
  const int m = i / (2 * rp), v = i - m * 2 * rp, j = v < rp ? v : v - rp;
  float s = 0.f;
  for (int z = 0; z < split; ++z) s += t[(size_t)z * tstride + (size_t)m * rp + j];
  const uint32_t hi = to16<BF16>(s);
  const float hif = BF16 ? __uint_as_float(hi << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)hi);
  t16[i] = (uint16_t)(v < rp ? hi : to16<BF16>(s - hif));
}

// A bitmap layer created for decode batches only (no dense int8 copy): row
// blocks of 32 through the decode kernels.
static hipError_t prefill_by_decode(const Layer& L, int M, const void* x, float* y, hipStream_t stream) {
  const int ldx = (x == L.xprep) ? L.Kx : L.h.K;
  for (int m0 = 0; m0 < M; m0 += kMaxDecodeM) {
    const int mb = M - m0 < kMaxDecodeM ? M - m0 : kMaxDecodeM;
    const void* xb = static_cast<const uint16_t*>(x) + (size_t)m0 * ldx;
    Layer Lb = L;
    if (x == L.xprep) Lb.xprep = const_cast<uint16_t*>(static_cast<const uint16_t*>(xb));
    // the bitmap format takes the matrix-core decode kernel (or, for a layer
    // without its workspace, the tile kernel); each block with a low-rank
    // prologue inside publishes an epoch (or generation) of its own
    const hipError_t e = launch_decode(Lb, mb, xb, y + (size_t)m0 * L.h.N, stream, 0);
    L.lr_epoch = Lb.lr_epoch;  // the copy took the next epochs
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_prefill(const Layer& L, int M, const void* x, float* y, hipStream_t stream) {
  const cl_blob_header& h = L.h;
  // the bitmap format: the INT8 tile loader over its dense int8 copy when the
  // layer was created for prefill batches, else the matrix-core decode in blocks
  const bool dense8 = L.pf_dense8 != nullptr;
  if (h.mask == CL_MASK_BITMAP && !dense8) return prefill_by_decode(L, M, x, y, stream);
  const bool bf16 = h.x_dtype == CL_ACT_BF16;
  PfArgs a = {};
  a.x = static_cast<const uint16_t*>(x);
  a.ldx = (x == L.xprep) ? L.Kx : h.K;
  a.M = M;
  a.K = h.K;
  const bool has_lr = h.lr != CL_LR_NONE && h.rank > 0;
  const int rp = L.pf_rp;
  hipError_t e = hipSuccess;
  if (has_lr) {
    // t = x' L on the matrix cores (L^T rows as the weight tile), split along K
    // so that the few output tiles of t still fill the chip
    PfArgs p = a;
    p.N = h.rank;
    p.Npad = h.rank;
    p.b16 = L.pf_l16;
    p.ldb16 = L.pf_Kl;
    p.nb16 = h.rank;
    p.y = L.t;
    p.ldy = rp;
    p.ncols = rp;
    p.nsteps = p.nsteps_dense = (int)ceil_div(L.pf_Kl, PfCfg<K_DENSE16>::bk);
    const int tiles = (int)(ceil_div(rp, kPfBN) * ceil_div(M, kPfBM));
    int split = (int)ceil_div(256, tiles);
    if (split > kPfMaxSplit) split = kPfMaxSplit;
    if (split > p.nsteps) split = p.nsteps;
    p.steps_per_split = (int)ceil_div(p.nsteps, split);
    split = (int)ceil_div(p.nsteps, p.steps_per_split);
    p.ystride = (size_t)M * rp;
    e = launch_prefill_kind<K_DENSE16>(p, bf16, stream);
    if (e != hipSuccess) return e;
    const int total = M * 2 * rp;
    if (bf16)
      hipLaunchKernelGGL(pf_tsplit_kernel<true>, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, stream, L.t,
                         p.ystride, split, M, rp, L.pf_t16);
    else
      hipLaunchKernelGGL(pf_tsplit_kernel<false>, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, stream, L.t,
                         p.ystride, split, M, rp, L.pf_t16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.a2 = L.pf_t16;
    a.lda2 = 2 * rp;
    a.r16 = L.pf_r16;
    a.ldr16 = 2 * rp;
  }
  a.N = h.N;
  a.Npad = L.Npad;
  a.dense = reinterpret_cast<const uint4*>(dense8 ? L.pf_dense8 : L.dense);
  a.meta = dense8 ? nullptr : L.meta;
  a.table = reinterpret_cast<const uint16_t*>(L.table);
  a.chunks = dense8 ? L.pf_chunks8 : h.chunks;
  a.cptr = L.pf_cptr;
  a.cent = L.pf_cent;
  a.y = y;
  a.ldy = h.N;
  a.ncols = h.N;
  a.ystride = 0;
  a.nsteps_dense = L.pf_nd;
  auto run = [&](auto kind_tag) {
    constexpr int KIND = decltype(kind_tag)::value;
    a.nsteps = a.nsteps_dense + (has_lr ? (int)ceil_div(2 * rp, PfCfg<KIND>::bk) : 0);
    a.steps_per_split = a.nsteps;
    if constexpr (KIND == K_LUT3) return launch_prefill_wide(a, bf16, stream);
    else return launch_prefill_kind<KIND>(a, bf16, stream);
  };
  switch (h.dense) {
    case CL_DENSE_LUT3: return run(std::integral_constant<int, K_LUT3>{});
    case CL_DENSE_LUT4: return run(std::integral_constant<int, K_LUT4>{});
    case CL_DENSE_INT4:
      return h.mask == CL_MASK_2_4 ? run(std::integral_constant<int, K_INT4_24>{}) : run(std::integral_constant<int, K_INT4>{});
    default: return run(std::integral_constant<int, K_INT8>{});
  }
}

}  // namespace cl
