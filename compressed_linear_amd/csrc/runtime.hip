// runtime.hip -- the C ABI: upload, forward dispatch, debug dequantisation.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "internal.h"
#include "layer.h"

namespace cl {

static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

// Split-K workgroups per tile: enough workgroups for about two per CU, each
// wave still streaming at least a few chunks.  CL_SPLIT overrides (tuning).
static int choose_split(const cl_blob_header& h, int num_cus) {
  const int forced = env_int("CL_SPLIT", 0);
  int s;
  if (forced > 0) {
    s = forced;
  } else {
    const int target = 2 * num_cus;
    s = (int)((target + h.n_tiles / 2) / h.n_tiles);
  }
  const int max_by_chunks = h.chunks / (4 * 2) > 0 ? h.chunks / (4 * 2) : 1;
  if (s > max_by_chunks) s = max_by_chunks;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return s;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t workspace_layout(const cl_blob_header& h, int32_t max_M, Layer* L, size_t base) {
  const int split = L ? L->split : 64;  // size query: the largest split
  const int Npad = h.n_tiles * 64;
  size_t off = align256(base);
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const int mblocks = (int)ceil_div(max_M, 32);
  const size_t o_cnt = take((size_t)(h.n_tiles + mblocks + 8) * 4);
  const size_t o_part = take((size_t)h.n_tiles * split * kMaxDecodeM * 64 * 4);
  size_t o_nzs = 0, o_t = 0, o_xp = 0;
  if (h.mask == CL_MASK_BITMAP) o_nzs = take((size_t)Npad * 4 * split * 4);
  if (h.lr != CL_LR_NONE && h.rank > 0) o_t = take((size_t)max_M * round_up(h.rank, 8) * 4);  // row stride <= rank rounded to 8
  // activations are restaged (clamped, row stride a multiple of 8 for aligned
  // 128-bit loads) when the layer clamps them or K is not a multiple of 8
  const int Kx = (int)round_up(h.K, 8);
  if (h.has_clamp || (h.K & 7)) o_xp = take((size_t)max_M * Kx * 2);
  if (L) {
    uint8_t* d = L->dev;
    L->counters = reinterpret_cast<uint32_t*>(d + o_cnt);
    L->part = reinterpret_cast<float*>(d + o_part);
    L->nzstart = o_nzs ? reinterpret_cast<int32_t*>(d + o_nzs) : nullptr;
    L->t = o_t ? reinterpret_cast<float*>(d + o_t) : nullptr;
    L->xprep = o_xp ? reinterpret_cast<uint16_t*>(d + o_xp) : nullptr;
    L->Kx = Kx;
    L->ws_bytes = off - align256(base);
  }
  return off;
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
  if (!dev_buf || reinterpret_cast<uintptr_t>(dev_buf) % 256) return fail(CL_EINVAL, "dev_buf must be 256-byte aligned");
  if (h->lr != CL_LR_NONE && h->rank > 256) return fail(CL_EUNSUPPORTED, "ranks above 256 are not built");
  Layer* L = new (std::nothrow) Layer();
  if (!L) return fail(CL_EINVAL, "out of host memory");
  L->h = *h;
  L->dev = static_cast<uint8_t*>(dev_buf);
  L->max_M = max_M;
  L->Npad = h->n_tiles * 64;
  int dev = 0;
  hipGetDevice(&dev);
  int cus = 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  L->num_cus = cus;
  L->split = choose_split(*h, cus);
  const size_t need = workspace_layout(*h, max_M, L, h->total_bytes);
  if (dev_bytes < need) {
    delete L;
    return fail(CL_ENOMEM, "dev_buf needs %zu bytes, got %zu", need, dev_bytes);
  }
  L->dev_bytes = dev_bytes;
  uint8_t* d = L->dev;
  L->dense = sec<uint8_t>(d, *h, CL_SEC_DENSE);
  L->table = sec<uint8_t>(d, *h, CL_SEC_TABLE);
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
  hipError_t e = hipMemcpyAsync(d, blob, h->total_bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemsetAsync(L->counters, 0, (size_t)(h->n_tiles + ceil_div(max_M, 32) + 8) * 4, s);
  if (e == hipSuccess && !nzs.empty())
    e = hipMemcpyAsync(L->nzstart, nzs.data(), nzs.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete L;
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
  if (path == CL_PATH_DECODE && M > kMaxDecodeM) return fail(CL_EINVAL, "the decode path takes M <= %d", kMaxDecodeM);
  if (path != CL_PATH_DECODE && path != CL_PATH_PREFILL) return fail(CL_EINVAL, "unknown path %d", path);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const void* xa = x;
  hipError_t e = hipSuccess;
  if (L->xprep) {
    e = launch_prep_x(*L, M, x, s);
    xa = L->xprep;
  }
  if (path == CL_PATH_DECODE) {
    if (e == hipSuccess && L->h.lr != CL_LR_NONE) e = launch_lowrank_prologue(*L, M, xa, s);
    if (e == hipSuccess) e = launch_decode(*L, M, xa, y, s);
  } else {
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
  delete static_cast<Layer*>(handle);
  return CL_OK;
}
