/*
 * compressed_linear.h -- C ABI of the MI355X (gfx950) compressed linear layer.
 *
 * The operation is the forward of one linear layer whose weight is stored
 * compressed:
 *
 *     y[m, n] = sum_k x'[m, k] * W_hat[n, k]        W_hat = D + S + (L_hat R_hat)^T
 *
 *   D      dense low-bit part, one row per output channel n:
 *            - 3- or 4-bit codes into a per-row table of fp16 centroids
 *              ("SqueezeLLM: Dense-and-Sparse Quantization", Approach: non-uniform
 *              LUT quantization with k-means centroids);
 *            - or symmetric int4 / int8 values times a per-row fp16 scale
 *              ("SLiM: One-shot Quantization and Sparsity with Low-rank
 *              Approximation for LLM Weight Compression", review highlights,
 *              SLiM-Quant: symmetric quantization, round to nearest);
 *            optionally under a 2:4 semi-structured or an unstructured mask
 *            (SLiM page, rebuttal "Unstructured vs. 2:4 Sparsity";
 *            "Compressing Large Language Models by Joint Sparsification and
 *            Quantization", Approach).
 *   S      outliers in CSR with fp16 values (SqueezeLLM page, Approach: the
 *          top-sensitivity and outlier weights, 0.45% in total, in a
 *          full-precision sparse matrix).
 *   L, R   low-rank correction (SLiM page, review highlights, SLiM-LoRA), fp16,
 *          bf16, or int4 with AbsMax group quantization, group 128 (SLiM page,
 *          review highlights, "Low-rank adapter quantization").
 *   x'     activations, clamped to [-c, c] when the layer carries a clamp c
 *          (JSQ page, Approach: activation editor with a per-layer strength).
 *
 * Conventions for every entry point:
 *   - Status codes are returned; nothing throws across the ABI.  The message of
 *     the last failure on the calling thread is returned by cl_last_error().
 *   - "host" pointers are CPU memory the caller owns; "device" pointers are GPU
 *     memory the caller owns (PyTorch allocates it in the Python binding).
 *     The library never frees caller memory and keeps no pointer to host
 *     arrays after a call returns.
 *   - Streams are hipStream_t values passed as void*; NULL means the default
 *     stream.  GPU work is asynchronous on that stream.
 *   - Every array is row-major and contiguous.  fp16 and bf16 values are
 *     passed as their uint16 bit patterns.
 */
#ifndef COMPRESSED_LINEAR_H
#define COMPRESSED_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CL_OK = 0,
  CL_EINVAL = -1,        /* malformed argument or layer description */
  CL_EUNSUPPORTED = -2,  /* valid, but a combination this library does not build */
  CL_ENOMEM = -3,        /* a caller buffer is too small */
  CL_EHIP = -4,          /* a HIP runtime call or kernel launch failed */
  CL_ESIZE = -5          /* a size exceeds the supported limits */
} cl_status;

typedef enum { CL_DENSE_LUT3 = 0, CL_DENSE_LUT4 = 1, CL_DENSE_INT4 = 2, CL_DENSE_INT8 = 3 } cl_dense_kind;
typedef enum { CL_MASK_NONE = 0, CL_MASK_2_4 = 1, CL_MASK_BITMAP = 2 } cl_mask_kind;
typedef enum { CL_LR_NONE = 0, CL_LR_FP16 = 1, CL_LR_BF16 = 2, CL_LR_INT4 = 3 } cl_lr_kind;
typedef enum { CL_ACT_F16 = 0, CL_ACT_BF16 = 1 } cl_act_dtype;
/* Forward paths: AUTO picks by M (decode for M <= 32, else prefill); DECODE
 * picks the faster decode kernel for M and the layer's shape; DECODE_VALU
 * forces the vector-ALU decode kernels (at M = 1 the row-wise one),
 * DECODE_MFMA the matrix-core decode kernel, DECODE_STREAM the batch-1
 * streaming kernel. */
typedef enum {
  CL_PATH_AUTO = 0,
  CL_PATH_DECODE = 1,
  CL_PATH_PREFILL = 2,
  CL_PATH_DECODE_VALU = 3,
  CL_PATH_DECODE_MFMA = 4,
  CL_PATH_DECODE_STREAM = 5
} cl_path;

/*
 * Logical (unpacked) description of one layer.  All pointers are host
 * pointers to arrays the caller owns; they are read only during cl_pack.
 * W_hat is [N, K]: N = out_features (rows), K = in_features.
 *
 *   dense = LUT3 / LUT4 : codes [N*K] uint8 in 0..2^b-1; lut [N * 2^b] fp16 bits,
 *                         the table of row n at lut[n * 2^b].
 *   dense = INT4 / INT8 : qvals [N*K] int8 (INT4: -8..7, INT8: -127..127);
 *                         row_scale [N] fp16 bits; D[n,k] = qvals[n,k] * row_scale[n].
 *   mask  = 2_4         : keep [N*K] 0/1, exactly two kept in each group of four
 *                         consecutive k (K % 4 == 0).  INT4 only (CL_EUNSUPPORTED otherwise).
 *   mask  = BITMAP      : keep [N*K] 0/1, any pattern.  INT8 only (CL_EUNSUPPORTED otherwise).
 *                         qvals at dropped positions are ignored.
 *   CSR                 : csr_row_ptr [N+1] int32 (row_ptr[0] = 0, nondecreasing,
 *                         row_ptr[N] = nnz), csr_col [nnz] int32 strictly
 *                         increasing within a row and < K, csr_val [nnz] fp16 bits.
 *                         nnz may be 0 (then the three pointers may be NULL).
 *   lr    = FP16 / BF16 : L [K*rank], R [rank*N] uint16 bit patterns.
 *   lr    = INT4        : L, R int8 codes in -8..7; L_scale [ceil(K/group) * rank]
 *                         (groups of `group` consecutive k per rank column),
 *                         R_scale [ceil(rank/group) * N] (groups along the rank
 *                         axis per output column), fp16 bits.
 *   has_clamp, act_clamp: x' = min(max(x, -c), c) with c = act_clamp (fp16 bits, c >= 0).
 *   x_dtype             : element type of x in cl_forward (fp16 or bf16).
 *   n_xscale, xscale_ch, xscale: per-channel activation scaling of SLiM's
 *                         output-error variant ("SLiM" page, rebuttal section "Output
 *                         Error Minimization in SLiM-Quant": the weights of a few
 *                         salient input channels carry a factor alpha, their
 *                         activations are divided by it while the layer runs).
 *                         The weights given above already include alpha.  xscale_ch
 *                         [n_xscale] int32, strictly increasing, < K; xscale
 *                         [n_xscale] fp16 bits of the activation factor f = 1/alpha,
 *                         a normal value in [2^-14, 1].  After the clamp,
 *                         x'[m, k] = x'[m, k] * f rounded once (nearest, ties to even)
 *                         to the activation type.  n_xscale = 0: no scaling (the two
 *                         pointers may be NULL).
 */
typedef struct {
  int32_t K, N;
  int32_t dense;            /* cl_dense_kind */
  int32_t mask;             /* cl_mask_kind */
  const uint8_t* codes;
  const uint16_t* lut;
  const int8_t* qvals;
  const uint16_t* row_scale;
  const uint8_t* keep;
  int64_t nnz;
  const int32_t* csr_row_ptr;
  const int32_t* csr_col;
  const uint16_t* csr_val;
  int32_t lr;               /* cl_lr_kind */
  int32_t rank;
  int32_t group;
  const void* L;
  const void* R;
  const uint16_t* L_scale;
  const uint16_t* R_scale;
  int32_t has_clamp;
  uint16_t act_clamp;
  uint16_t reserved0;
  int32_t x_dtype;          /* cl_act_dtype */
  int32_t n_xscale;
  const int32_t* xscale_ch;
  const uint16_t* xscale;
} cl_layer_desc;

/*
 * Canonical byte accounting of a packed layer: what the method must move per
 * forward, independent of device padding.
 *   codes        LUT3: N*ceil(K/10)*4 (ten 3-bit codes per 32-bit word, each row
 *                starting a new word); LUT4 / INT4: N*ceil(K/8)*4; INT8: N*K;
 *                masked INT: the kept values only (2:4: N*K/2 values).
 *   lut_or_scale N * 2^b * 2 (LUT) or N * 2 (per-row scales)
 *   mask_meta    2:4: 2 bits per kept value (N*K/8 bytes); BITMAP: N*ceil(K/32)*4
 *                bitmap words plus (N+1)*4 bytes of nonzero offsets.
 *   csr          6*nnz + 4*(N+1)
 *   lowrank      factor bytes (2 per value; int4: 1/2 per value) plus scales
 *   act_scale    6 per scaled input channel (int32 channel, fp16 factor)
 *   total        the sum of the above
 *   device_padding  extra bytes of the device layout (row and tile padding),
 *                   not part of `total`.
 */
typedef struct {
  uint64_t codes, lut_or_scale, mask_meta, csr, lowrank, act_scale, total;
  uint64_t device_padding;
} cl_bytes;

/*
 * cl_pack -- validate a layer description and lay it out for the device.
 *   desc        host, read only.
 *   blob        host output buffer of *blob_bytes bytes, 16-byte aligned; NULL
 *               asks for the size only.
 *   blob_bytes  in: capacity of blob; out: bytes needed / written.
 *   acct        host, optional (NULL): canonical byte accounting.
 * Host only; never touches a GPU.  Errors: CL_EINVAL for malformed input
 * (shapes, code or value ranges, a 2:4 group without exactly two kept, CSR
 * pointers not nondecreasing, columns out of range, unsorted or repeated),
 * CL_EUNSUPPORTED for combinations not built (a mask on a LUT format, a
 * 2:4 mask with K % 4 != 0), CL_ESIZE for dimensions above 2^24,
 * nnz above 2^31 - 1, or a section of the device layout of 2^31 bytes or
 * more (checked from the dimensions before any array is read; the kernels
 * address each buffer through a 32-bit range), CL_ENOMEM if *blob_bytes is
 * too small.
 * The blob is self-describing (it starts with a cl_blob_header) and may be
 * saved and reloaded byte for byte.
 */
cl_status cl_pack(const cl_layer_desc* desc, void* blob, size_t* blob_bytes, cl_bytes* acct);

/*
 * cl_device_bytes -- device memory (bytes) that cl_create needs for `blob`
 * with forwards of up to max_M activation rows: the packed layer plus the
 * workspace (split-K partial sums, counters, the low-rank intermediate
 * x' L_hat, restaged activations) and the data the matrix-core path derives
 * at create (outlier lists per 128-row tile and K step, the low-rank factors
 * in the 16-bit MFMA input type; for a bitmap layer with max_M > 32, a dense
 * int8 copy of its weights, N*K bytes rounded up, zero where dropped, that the
 * prefill's matrix-core tile loader reads).  Returns 0 if the blob is
 * malformed (the reason in cl_last_error), max_M < 1, or a workspace buffer or
 * the activations of max_M rows would take 2^31 bytes or more.
 *
 * Blob checks (here and in cl_create), on the host: the header fields agree
 * with each other; every section has the length the header implies and lies
 * inside total_bytes (overflow-safe); the CSR row pointers run from 0 to nnz
 * without decreasing and each row's columns increase strictly below K; the
 * bitmap's row offsets are multiples of 16 that hold each row's kept values
 * inside its section, and padding rows keep nothing.  The blob buffer must
 * hold total_bytes bytes (a blob written by cl_pack does).
 */
size_t cl_device_bytes(const void* blob, int32_t max_M);

/*
 * cl_create -- upload a packed layer to the current HIP device.
 *   blob      host, read during the call (the copy is synchronised before
 *             return, so the caller may free it afterwards).
 *   dev_buf   device, at least cl_device_bytes(blob, max_M) bytes, 256-byte
 *             aligned, owned by the caller, must outlive the handle.
 *   max_M     largest M a later cl_forward will pass.
 *   stream    hipStream_t for the upload, the workspace clear and the
 *             derived tables (built on the host from the blob, then copied).
 *   handle    out: opaque handle (host memory owned by the library).
 * Errors: CL_EINVAL (malformed blob, see cl_device_bytes; NULL or misaligned
 * pointers), CL_ESIZE (a workspace buffer or the activations of max_M rows
 * at 2^31 bytes or more), CL_ENOMEM (dev_bytes too small), CL_EHIP (copy failed).
 */
cl_status cl_create(const void* blob, void* dev_buf, size_t dev_bytes, int32_t max_M,
                    void* stream, void** handle);

/*
 * cl_forward -- y = x' W_hat^T for M rows of activations.
 *   x_dev  device, [M, K] fp16 or bf16 (the layer's x_dtype), 16-byte aligned;
 *          read only (the clamp and the channel scaling, if the layer has them,
 *          go to a copy in the workspace or are applied while staging).
 *   y_dev  device, [M, N] fp32, overwritten, 16-byte aligned.
 *   1 <= M <= max_M.  M <= 32 runs the decode kernels (the vector-ALU
 *   streaming kernel at small M, the matrix-core decode kernel with weights
 *   dequantised in registers at larger M); larger M runs the prefill kernels
 *   (MFMA on dequantised LDS tiles).
 * One forward at a time per handle (the workspace inside dev_buf is shared).
 * A forward may be recorded into a HIP graph and replayed: the kernels keep
 * their own state on the device (counters return to zero, and a launch that
 * computes x' L_hat inside derives its generation from device memory), so no
 * argument changes between replays.
 * Deterministic: the same inputs give bitwise identical y.
 * The layer's own low-rank prologue runs inside the decode launch where it
 * can: its waits for x' L_hat are bounded, and one that gives up (see
 * cl_set_wait_limit) leaves NaN in the outputs it could not finish.
 * Errors: CL_EINVAL (M out of range, NULL or misaligned pointers),
 * CL_EHIP (launch failure; or an earlier forward's wait gave up -- reported
 * once, and this call then launches nothing).
 */
cl_status cl_forward(void* handle, int32_t M, const void* x_dev, float* y_dev, void* stream);

/* cl_forward with an explicit path (cl_path); CL_PATH_AUTO behaves as cl_forward.
 * The decode paths require M <= 32; CL_PATH_DECODE_MFMA also a bitmap layer or
 * one created with max_M >= 2, CL_PATH_DECODE_STREAM M = 1 and a layer whose
 * shape fits the streaming kernel's LDS plan (else CL_EUNSUPPORTED). */
cl_status cl_forward_path(void* handle, int32_t M, const void* x_dev, float* y_dev,
                          void* stream, int32_t path);

/*
 * cl_debug_dequant -- write the dequantised parts of W_hat with the same
 * unpacking device code the forward uses (a parity aid; not timed).
 *   D16  device, [N, K] fp16: D, zero where masked (integer formats: q*s
 *        rounded once to fp16, nearest-even).
 *   S16  device, [N, K] fp16: the CSR outliers at their positions, else 0.
 *   L32  device, [K, rank] fp32 and R32 device, [rank, N] fp32 (exact); may
 *        be NULL, and are ignored for a layer without a low-rank part.
 * Errors: CL_EINVAL (NULL D16 / S16), CL_EHIP.
 */
cl_status cl_debug_dequant(void* handle, uint16_t* D16, uint16_t* S16, float* L32, float* R32,
                           void* stream);

/* cl_destroy -- free the host handle (and its pinned error word).  The caller
 * frees dev_buf afterwards. */
cl_status cl_destroy(void* handle);

/*
 * cl_set_wait_limit -- test support for the failure path of the low-rank
 * prologue inside a decode launch ("SLiM" page, review highlights: y gets the
 * term (x' L_hat) R_hat).  A batch-1..32 forward of a layer with a low-rank
 * part computes t = x' L_hat in the launch's first workgroups and publishes
 * it; the workgroups that add the rank term wait for it, polling a bounded
 * number of times.
 *   handle     from cl_create.
 *   max_polls  bound of that wait, in polls of a few hundred cycles after the
 *              first look (cl_create sets 2^20, far above any producer's time).
 *   withhold   nonzero: the prologue computes t but does not publish it, so
 *              every wait runs to its bound and every kernel still ends.
 * A wait that gives up writes NaN to the outputs that needed t and sets the
 * layer's error word (pinned host memory); the next cl_forward on the handle
 * then returns CL_EHIP, once, without launching anything.
 * Errors: CL_EINVAL (NULL handle).
 */
cl_status cl_set_wait_limit(void* handle, uint32_t max_polls, int32_t withhold);

/* Message of the last failing call on this thread ("" if none). */
const char* cl_last_error(void);

/*
 * cl_fit_lut_work_bytes -- device scratch (bytes) that cl_fit_lut needs for an
 * N x K matrix; 0 if N or K < 1.
 */
size_t cl_fit_lut_work_bytes(int32_t N, int32_t K);

/*
 * cl_fit_lut -- data-free LUT packing of an fp16 weight matrix on the GPU, the
 * step before cl_pack ("SqueezeLLM: Dense-and-Sparse Quantization", Approach:
 * per-output-channel non-uniform LUTs from k-means, outliers to a
 * full-precision CSR matrix; the sensitivity-agnostic variant of its
 * measured-effects table, from weights alone).
 *   W         device, [N, K] fp16 weights, row = output channel; finite,
 *             |w| < 8192.
 *   bits      3 or 4 (LUTs of 8 or 16 values).
 *   n_out     weights moved to the CSR part: the n_out of largest magnitude,
 *             ties to the lower row-major index (0 <= n_out <= N*K, < 2^31).
 *   max_iter  Lloyd iterations per row at most (>= 1); a row stops when no
 *             centroid moves.  Row n starts from 2^b points spread evenly over
 *             [min, max] of its dense weights: c_j = min + (max-min)(2j+1)/2^(b+1);
 *             a weight joins the nearest centroid (the lower on a tie); a
 *             centroid becomes the mean of its weights (kept when it has none).
 *   outputs (device, caller-owned): codes [N*K] uint8 (nearest LUT value, the
 *             lower code on a tie; an outlier's position takes the code nearest
 *             to 0); lut [N * 2^b] fp16 (the centroids rounded to nearest-even);
 *             row_ptr [N+1] int32, col [n_out] int32 (ascending in each row),
 *             val [n_out] fp16 = fp16(w - lut[code]) -- exactly the logical
 *             arrays cl_pack takes for a LUT layer with CSR outliers.
 *   work      device, cl_fit_lut_work_bytes(N, K) bytes, 8-byte aligned.
 *   stream    hipStream_t; the call synchronizes it before returning.
 *   total_iters  host, optional (NULL): the Lloyd iterations run, summed over rows.
 * Deterministic: cluster sums are exact integers (weights are multiples of
 * 2^-24), every other decision exact or rounded once in a fixed order.
 * Errors: CL_EINVAL (sizes, bits, n_out, max_iter, NULL pointers, or a weight
 * that is not finite or has |w| >= 8192: outputs then undefined), CL_ESIZE
 * (K > 28672 or N > 2^24), CL_EHIP.
 */
cl_status cl_fit_lut(const uint16_t* W, int32_t N, int32_t K, int32_t bits, int64_t n_out, int32_t max_iter,
                     uint8_t* codes, uint16_t* lut, int32_t* row_ptr, int32_t* col, uint16_t* val,
                     void* work, void* stream, int64_t* total_iters);

/*
 * cl_fit_lut_noalloc -- cl_fit_lut for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same kernels and outputs, with the work buffer
 * replaced by a scratch array of 2 MiB that the library holds on every device
 * it runs on until the process ends (static device memory; this call
 * allocates nothing and calls no allocating routine).
 *   Arguments as cl_fit_lut, without `work`; N <= 130972 rows (the scratch
 *   holds 1600 + 16 N bytes).
 * Calls on one device share that scratch: calls that overlap on one device
 * (other streams, other threads) race and give undefined outputs; calls in
 * sequence are independent (each clears what must start at zero).  Like
 * cl_fit_lut it waits for its stream before returning.
 * Errors: those of cl_fit_lut; CL_ESIZE also for N above 130972;
 * CL_EUNSUPPORTED for a device index of 64 or more.
 */
cl_status cl_fit_lut_noalloc(const uint16_t* W, int32_t N, int32_t K, int32_t bits, int64_t n_out, int32_t max_iter,
                             uint8_t* codes, uint16_t* lut, int32_t* row_ptr, int32_t* col, uint16_t* val,
                             void* stream, int64_t* total_iters);

/*
 * cl_fit_int -- data-free packing of an fp16 weight matrix into the integer
 * formats on the GPU, the step before cl_pack ("SLiM" page, review highlights:
 * symmetric quantization that clips the weights before rounding to nearest,
 * the clipping threshold found by a grid search -- its probabilistic
 * formulation has no equations on the page, read as the plain squared error;
 * rebuttal "Unstructured vs. 2:4 Sparsity" and "Compressing Large Language
 * Models by Joint Sparsification and Quantization", Approach: 2:4 and
 * unstructured masks, here by magnitude since activation-aware metrics need data).
 *   W          device, [N, K] fp16 weights (finite), row = output channel.
 *   bits       4 (codes -7..7) or 8 (-127..127): qmax = 2^(bits-1) - 1.
 *   mask       CL_MASK_NONE; CL_MASK_2_4 (bits 4, K % 4 == 0): the two largest
 *              |w| of each group of four consecutive weights; CL_MASK_BITMAP
 *              (bits 8): the floor(K/2) largest |w| of each row.  Ties go to
 *              the lower index.
 *   grid       G in [1, 4096]: per row, the scale candidates
 *              s_i = fp16((i * max|w_kept|) / (qmax * G)), i = 1..G (fp64 division,
 *              nearest-even fp16); codes q = clamp(rint(w / s_i), -qmax, qmax);
 *              the candidate with the smallest sum of (w - s_i q)^2 over the kept
 *              weights (exact: a 128-bit integer in units of 2^-48) wins, the lower
 *              i on a tie.  A row with nothing kept or no positive candidate gets
 *              scale 0 and codes 0.
 *   outputs (device, caller-owned): qvals [N*K] int8 (0 where dropped),
 *              row_scale [N] fp16, keep [N*K] uint8 0/1 (may be NULL without a
 *              mask) -- the logical arrays cl_pack takes for the integer formats.
 *   work       device, 8 bytes, 8-byte aligned.
 *   stream     hipStream_t; the call synchronizes it before returning.
 * Errors: CL_EINVAL (sizes, bits, grid, NULL pointers, a weight that is not
 * finite: outputs then undefined), CL_EUNSUPPORTED (a mask with the other bit
 * width, 2:4 with K % 4 != 0), CL_ESIZE (K > 28672 or N > 2^24), CL_EHIP.
 */
cl_status cl_fit_int(const uint16_t* W, int32_t N, int32_t K, int32_t bits, int32_t mask, int32_t grid,
                     int8_t* qvals, uint16_t* row_scale, uint8_t* keep, void* work, void* stream);

/*
 * cl_quant_absmax -- AbsMax int4 group quantization of a low-rank factor on the
 * GPU ("SLiM" page, review highlights: the adapters are quantized with an AbsMax
 * group scheme, group size 128), the step before cl_pack for CL_LR_INT4.
 *   F       device, [R, C] fp16 values (bf16 = 0) or bf16 bit patterns (bf16 = 1),
 *           finite; L is passed as [K, r], R as [r, N].
 *   group   groups of `group` consecutive entries along the first axis, per column
 *           (the last one ragged).
 *   q       device, [R, C] int8 codes: clamp(rint(v / scale), -8, 7) in fp64.
 *   scale   device, [ceil(R / group), C] fp16: fp16(max|v| / 7) of the group (fp64
 *           division, nearest-even); 0 for an all-zero group (its codes 0) --
 *           the L_scale / R_scale layouts cl_pack takes.
 *   stream  hipStream_t; asynchronous.
 * Errors: CL_EINVAL (sizes, NULL pointers), CL_ESIZE, CL_EHIP.
 */
cl_status cl_quant_absmax(const uint16_t* F, int32_t R, int32_t C, int32_t group, int32_t bf16, int8_t* q,
                          uint16_t* scale, void* stream);

/*
 * cl_fit_lowrank -- Naive-LoRA ("SLiM" page, review highlights, SLiM-LoRA
 * bullet: the low-rank part that minimises the plain error norm between the
 * original and the compressed weight matrix): factors L, R of rank `rank`
 * such that (L R)^T approximates the truncated SVD of the residual
 * E = W - W_hat, found by randomized subspace iteration (rocBLAS products on
 * the GPU, m x m eigenproblems on the host; m = min(rank + oversample, N, K)).
 * The singular values are split evenly: L = V_r diag(sqrt(s)), R = diag(sqrt(s))
 * U_r^T.  The factors are fp32; cast them (or quantize with cl_quant_absmax)
 * for cl_pack.
 *   E           device, [N, K] fp32 row-major (rows = output channels), finite.
 *   rank        1..512; ranks past min(N, K) get zero factors.
 *   oversample  extra columns of the search subspace (>= 0; 16 is a good start).
 *   iters       power iterations, 0..100 (each one: two products with E).
 *   seed        of the Gaussian start matrix (the result depends on it only
 *               through rounding once the iteration has converged).
 *   L           device, [K, rank] fp32 row-major; R device, [rank, N] fp32.
 *   sigma       host, [rank] fp32 singular-value estimates (descending), or NULL.
 *   stream      hipStream_t; the call returns when the factors are written.
 * Allocates its work matrices (about 4 (N + K) m + 8 m^2 bytes).
 * Errors: CL_EINVAL (sizes, NULL pointers), CL_ESIZE (2^31 elements or bytes
 * in E or a work matrix), CL_ENOMEM, CL_EHIP.
 */
cl_status cl_fit_lowrank(const float* E, int32_t N, int32_t K, int32_t rank, int32_t oversample, int32_t iters,
                         uint64_t seed, float* L, float* R, float* sigma, void* stream);

/*
 * Header at the start of every packed blob (little endian).  Exposed so that
 * tools can inspect a blob; the section layouts are documented with the
 * packer.
 */
#define CL_BLOB_MAGIC 0x31424C43u /* "CLB1" */
#define CL_BLOB_VERSION 2u
enum {
  CL_SEC_DENSE = 0,   /* dense stream, row-major 16-byte chunks (bitmap: kept values) */
  CL_SEC_TABLE,       /* LUT [Npad * 2^b] fp16 or row scales [Npad] fp16 */
  CL_SEC_META,        /* 2:4 metadata or bitmap words, row-major chunks */
  CL_SEC_NZOFF,       /* BITMAP: int32 [N+1] start of each row's kept values */
  CL_SEC_ROWPTR,      /* CSR row_ptr int32 [N+1] */
  CL_SEC_COL,         /* CSR col int32 [nnz] */
  CL_SEC_VAL,         /* CSR val fp16 [nnz] */
  CL_SEC_L,           /* low-rank L, transposed: [rank][K] */
  CL_SEC_R,           /* low-rank R, transposed: [Npad][rank] */
  CL_SEC_LSCALE,      /* int4 L scales, [rank][ceil(K/group)] */
  CL_SEC_RSCALE,      /* int4 R scales, [Npad][ceil(rank/group)] */
  CL_SEC_XSCALE,      /* activation factors fp16 [K], 1 on the unscaled channels */
  CL_SEC_COUNT = 16
};
typedef struct {
  uint32_t magic, version;
  int32_t K, N, dense, mask, lr, rank, group, x_dtype, has_clamp;
  uint16_t act_clamp, reserved0;
  int32_t n_tiles;       /* ceil(N / 64) */
  int32_t chunks;        /* 16-byte chunks per row in the dense stream */
  int32_t span;          /* logical k covered by one chunk */
  int32_t meta_chunk_bytes; /* bytes of META per row per chunk (0 if none) */
  int64_t nnz;
  uint64_t total_bytes;  /* size of the whole blob */
  uint64_t off[CL_SEC_COUNT];
  uint64_t len[CL_SEC_COUNT];
  cl_bytes acct;
  int32_t n_xscale;      /* scaled input channels */
  uint8_t reserved[60];
} cl_blob_header;

#ifdef __cplusplus
}
#endif
#endif /* COMPRESSED_LINEAR_H */
