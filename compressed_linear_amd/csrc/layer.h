// layer.h -- the host-side handle of an uploaded layer and the launch entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "compressed_linear.h"
#include "layout.h"

namespace cl {

constexpr int kMaxDecodeM = 32;
constexpr int kLrSlice = 512;  // K rows per workgroup of the decode low-rank prologue
constexpr uint32_t kLrMaxPolls = 1u << 20;  // default bound of the in-launch wait for t (polls)

// Launch plan of the batch-1 streaming kernel, made at create (ok = 0: the
// row-wise kernel serves batch 1).  LDS offsets are bytes into the dynamic LDS.
struct StreamPlanH {
  int ok = 0;    // the layer fits the kernel's plan
  int pick = 0;  // and the kernel is the faster batch-1 choice for its shape
  int wpg = 0, rows_per_wg = 0, nwg = 0, lds = 0, out_cap = 0;
  int lds_x = 0, lds_max = 0, lds_meta = 0, lds_rp = 0, lds_rank = 0, lds_rsc = 0, lds_part0 = 0, lds_part1 = 0, lds_out = 0, lds_t = 0;
  int rank_row_bytes = 0, rank_row_stride = 0, rsc_row_bytes = 0;
  int lr_nl = 1;  // int4 prologue: 16-byte loads a thread of a 1024-thread block
};

struct Layer {
  cl_blob_header h;          // copy of the blob header
  uint8_t* dev = nullptr;    // dev_buf (caller owned)
  size_t dev_bytes = 0;
  int32_t max_M = 0;
  int Npad = 0;
  int split = 1;             // split-K workgroups per tile (decode)
  int num_cus = 256;

  // packed sections on the device (NULL when absent)
  const uint8_t* dense = nullptr;
  const uint8_t* table = nullptr;
  const uint8_t* meta = nullptr;
  const int32_t* nzoff = nullptr;
  int32_t* nzstart = nullptr;    // bitmap: [Npad][4*split] (workspace, filled at create)
  const int32_t* rowptr = nullptr;
  const int32_t* col = nullptr;
  const uint16_t* val = nullptr;
  const uint8_t* L = nullptr;
  const uint8_t* R = nullptr;
  const uint16_t* Lscale = nullptr;
  const uint16_t* Rscale = nullptr;

  // workspace (inside dev_buf, after the packed sections)
  uint32_t* counters = nullptr;  // [n_tiles + 1], zero between forwards
  float* part = nullptr;         // [n_tiles][split][kMaxDecodeM][64]
  float* t = nullptr;            // [max_M][rank]
  uint16_t* xprep = nullptr;     // [max_M][Kx]  clamped / scaled / padded activations
  const uint16_t* xscale = nullptr;  // [K] fp16 per-channel activation factors (1 where unscaled), or null
  int Kx = 0;                    // row stride of xprep (even)

  // matrix-core prefill (built at create)
  int pf_nd = 0;                 // K steps over the packed weights
  uint8_t* pf_dense8 = nullptr;  // bitmap layers created for prefill: dense INT8 chunk stream (zero where dropped)
  int pf_chunks8 = 0;            // its 16-byte chunks per row
  int32_t* pf_cptr = nullptr;    // outliers per (128-row tile, step): offsets [n_tiles128][pf_nd + 1]
  uint32_t* pf_cent = nullptr;   // entries: row in tile | k in step << 7 | fp16 value << 16
  uint16_t* pf_r16 = nullptr;    // [Npad][2 rp]: R^T twice, in the MFMA input type
  uint16_t* pf_l16 = nullptr;    // [rank][Kl]: L^T, rows padded to Kl = K rounded up to 8, MFMA input type
  uint16_t* pf_t16 = nullptr;    // [max_M][2 rp]: t_hi | t_lo of t = x' L (workspace)
  int pf_rp = 0, pf_Kl = 0;

  // decode low-rank prologue t = x' L, split over K (built at create); lr_mode
  // -1: the per-column kernel (L type differs from x, or int4 groups below 16),
  // 0: 16-bit L of the activation type, 1: int4 L
  int lr_mode = -1;
  int lr_rpad = 0;               // rank rounded up to 64
  int lr_S = 0;                  // K slices of kLrSlice rows
  uint8_t* lr_lk = nullptr;      // L, k-major in k pairs: 16-bit [Kl/2][rpad][2]; int4 bytes [Kl/2][rpad] (k even low nibble)
  uint16_t* lr_ls = nullptr;     // int4: scales k-major [ceil(Kl/group)][rpad]
  float* lr_part = nullptr;      // partial sums [tiles][S][256] (tagged 64-bit words in the streaming kernel)
  size_t lr_part_bytes = 0;
  mutable uint32_t lr_epoch = 0; // epochs of direct calls with the prologue inside (never 0)
  uint32_t* lr_cnt = nullptr;    // [kLrCntWords]: arrivals per output tile [0, 64), completed tiles [64],
                                 // published epoch [65], published generation [66], finished
                                 // generation [67], finished reader slots [68], reader slots at
                                 // 128 + 32 j (j < 32); counters zero between forwards

  // matrix-core decode (batch 2..32; absent when max_M == 1)
  int mf_npw = 0, mf_Kz = 0, mf_S = 0, mf_tiles = 0;
  float* mf_part = nullptr;      // slice partial sums [tiles][S][32][128]
  int32_t* mf_ooff = nullptr;    // outlier offsets per (slice, tile, row in tile): [S * tiles * 128 + 1]
  uint32_t* mf_oent = nullptr;   // entries: k in slice | fp16 value << 16
  int32_t* mf_nzs = nullptr;     // bitmap: first kept byte of every (row, slice) [Npad][S]
  size_t ws_bytes = 0;

  // waits for t inside a launch: poll bound, the error word a wait that gives
  // up sets (pinned host memory, so the next forward reads it without a sync;
  // wait_err_dev is its device address), and the test switch that withholds
  // the publication of t
  StreamPlanH st;                // batch-1 streaming kernel
  uint32_t wait_polls = 0;
  int wait_withhold = 0;
  volatile uint32_t* wait_err_host = nullptr;
  uint32_t* wait_err_dev = nullptr;
};

// Workspace layout and size for a blob header (used by cl_device_bytes and cl_create).
// *largest (optional) receives the size of the largest single workspace buffer.
size_t workspace_layout(const cl_blob_header& h, int32_t max_M, Layer* L /* may be NULL */, size_t base,
                        size_t* largest = nullptr);

// Kernel launchers (kernels.hip).  All asynchronous on `stream`.
hipError_t launch_prep_x(const Layer& L, int M, const void* x, hipStream_t stream);
hipError_t launch_lowrank_prologue(const Layer& L, int M, const void* x, hipStream_t stream);
// decode forward (M <= kMaxDecodeM), including the activation clamp / restaging
// (x: the caller's activations, or L.xprep when done already) and the low-rank
// prologue: inside the decode launch when it applies (publishing the launch's
// generation, derived on the device), else as kernels of their own.
// variant: 0 the faster kernel for M, 1 the vector-ALU kernels (row-wise at M = 1),
// 2 the matrix-core kernel, 3 the batch-1 streaming kernel (M = 1, st.ok)
hipError_t launch_decode(const Layer& L, int M, const void* x, float* y, hipStream_t stream, int variant);
hipError_t launch_prefill(const Layer& L, int M, const void* x, float* y, hipStream_t stream);
// Plan of the batch-1 streaming kernel from the blob header and its CSR row
// pointers (NULL without outliers), for a device of num_cus CUs.
StreamPlanH plan_stream(const cl_blob_header& h, const int32_t* rowptr, int num_cus, int lr_mode);
hipError_t launch_debug(const Layer& L, uint16_t* D16, uint16_t* S16, float* L32, float* R32, hipStream_t stream);

}  // namespace cl
