// lowrank.h -- the low-rank prologue t = x' L_hat split over K (one workgroup's
// share), used by its own kernel and inside the batch-1..4 decode kernel.
#pragma once
#include <hip/hip_runtime.h>

#include "layer.h"
#include "unpack.h"

namespace cl {

// ---------------------------------------------------------------------------
// The same t = x' L_hat split over K: workgroup (s, tj, tm) takes K rows
// [512 s, 512 s + 512), rank columns [64 tj, 64 tj + 64) and activation rows
// [MT tm, MT tm + MT), reading the k-major copy of L with 16-byte loads (all
// issued before any arithmetic).  Its partial sums go to memory; the last
// workgroup of each (tj, tm) tile to arrive adds the slices in slice order and
// stores t, so the result does not depend on arrival order.  The same block
// code runs as its own kernel (lr_split_kernel) or as the first workgroups of
// the batch-1..4 decode kernel, whose row workgroups wait for the published t.
//   MODE 0: 16-bit L of the activation type; a 16-byte load holds (k, k+1)
//           for 4 columns, consumed by pairwise dot products with (x_k, x_k+1).
//   MODE 1: int4 L; a 16-byte load holds (k, k+1) for 16 columns; each value
//           is q * s in fp32 (exact), s from the slice's scale rows in LDS.
// ---------------------------------------------------------------------------
struct LrSplitArgs {
  const uint16_t* x;
  int ldx, M, rank, rpad, S, group, Kl;
  const uint8_t* lk;
  const uint16_t* ls;
  float* part;
  uint32_t* cnt;      // arrivals per (tj, tm) tile
  float* t;
  // inside the decode kernel only (NULL otherwise): the workgroup that
  // completes the last tile publishes the launch's epoch (or, for epoch 0, its
  // generation; see lr_target) once every t value of the forward is in memory;
  // `done` counts completed tiles
  uint32_t* done;
  uint32_t* flag;
  uint32_t epoch;
  int ntiles;
  int withhold;       // test support: compute t but never publish it (every reader's wait then gives up)
  // clamp x to [-cval, cval] and multiply it by the per-channel factors
  // xscale ([K] fp16, NULL: none) while staging it (raw activations only)
  int clamp;
  float cval;
  const uint16_t* xscale;
};

// Activation editor of "Compressing Large Language Models by Joint
// Sparsification and Quantization" (Approach: one clamp value per layer),
// applied to eight staged 16-bit activations.  +-c is exact in the activation
// type (checked by the packer), so the clamped value is the input or +-c
// exactly, as when the activations are clamped by a kernel of their own.
template <bool BF16>
__device__ __forceinline__ uint4 clamp_act8(uint4 v, float c) {
  uint32_t u[4] = {v.x, v.y, v.z, v.w};
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = fminf(fmaxf(__uint_as_float(u[i] << 16), -c), c);
      const float hi = fminf(fmaxf(__uint_as_float(u[i] & 0xFFFF0000u), -c), c);
      u[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
  } else {
    const half2_t hc = {(_Float16)c, (_Float16)c}, lc = {(_Float16)-c, (_Float16)-c};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = as_u32(__builtin_elementwise_min(__builtin_elementwise_max(as_h2(u[i]), lc), hc));
  }
  return make_uint4(u[0], u[1], u[2], u[3]);
}

// fp32 -> bf16, nearest with ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Per-channel activation factors of SLiM's output-error variant ("SLiM" page,
// rebuttal section "Output Error Minimization in SLiM-Quant": the activations
// of the salient channels are divided by alpha; the layer stores f = 1/alpha,
// 1 elsewhere), applied to eight staged 16-bit activations with their eight
// fp16 factors.  The product is rounded once to the activation type, nearest
// with ties to even: an fp16 multiply does exactly that; for bf16 the product
// of a bf16 and an fp16 value is exact in fp32 (8 + 11 significant bits) and
// is rounded from there.
template <bool BF16>
__device__ __forceinline__ uint4 scale_act8(uint4 v, uint4 f) {
  uint32_t u[4] = {v.x, v.y, v.z, v.w};
  const uint32_t g[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BF16) {
      const float lo = __uint_as_float(u[i] << 16) * (float)__builtin_bit_cast(_Float16, (uint16_t)(g[i] & 0xFFFFu));
      const float hi = __uint_as_float(u[i] & 0xFFFF0000u) * (float)__builtin_bit_cast(_Float16, (uint16_t)(g[i] >> 16));
      u[i] = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
    } else {
      u[i] = as_u32(as_h2(u[i]) * as_h2(g[i]));
    }
  }
  return make_uint4(u[0], u[1], u[2], u[3]);
}

// Publication of t by a prologue inside a decode launch.  Words of the
// counters from `flag` (word 65) on: [0] the epoch published by the last
// launch called directly (the host passes a new epoch each call), [1] the
// generation published by the last launch recorded into a graph, [2] gen, the
// generation of the last recorded launch whose readers of t have all finished,
// [3] the count of finished reader slots; from word 128 on, kLrSlots slot
// counters of finished readers, one per 128-byte line (atomics on one line
// serialize).  A recorded launch gets epoch 0 and derives its generation,
// gen + 1, on the device, so that a replay needs no new argument: gen only
// moves when the launch's last reader is done, so every workgroup of the
// launch reads the same value.  The two kinds keep separate words, so direct
// calls and replays can interleave.
constexpr int kLrSlots = 32;
__device__ __forceinline__ uint32_t lr_target(const uint32_t* flag, uint32_t epoch) {
  return epoch ? epoch
               : __hip_atomic_load(const_cast<uint32_t*>(flag) + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
}
__device__ __forceinline__ uint32_t* lr_word(const uint32_t* flag, uint32_t epoch) {
  return const_cast<uint32_t*>(flag) + (epoch ? 0 : 1);
}

// Recorded launches: one call per reader of t (reader `idx` of `readers`) after
// its last read of t; the last one of the launch moves gen on.
__device__ __forceinline__ void lr_reader_done(uint32_t* flag, uint32_t generation, int readers, int idx) {
  const int j = idx % kLrSlots;
  const int share = readers / kLrSlots + (j < readers % kLrSlots ? 1 : 0);
  const int used = readers < kLrSlots ? readers : kLrSlots;
  uint32_t* slot = flag - 65 + 128 + 32 * j;
  if (__hip_atomic_fetch_add(slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(share - 1)) {
    __hip_atomic_store(slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__hip_atomic_fetch_add(flag + 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(used - 1)) {
      __hip_atomic_store(flag + 3, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(flag + 2, generation, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Bounded wait for the published t.  Lane 0 polls `word` (each poll sleeps a
// few hundred cycles) at most max_polls times after the first look; the
// default bound, far above any producer's run time, only keeps a wavefront
// from waiting forever should a producer never publish (its progress rests on
// the producers being dispatched before the readers, the launch's first
// workgroups).  A wait that gives up records it in the layer's error word
// (host memory, read by the next forward) and returns false for the whole
// wavefront: the caller then writes NaN instead of using a stale t.
__device__ __forceinline__ bool wait_lowrank(const uint32_t* word, uint32_t target, int lane, uint32_t max_polls,
                                             uint32_t* err) {
  int ok = 1;
  if (lane == 0) {
    uint32_t it = 0;
    while (__hip_atomic_load(const_cast<uint32_t*>(word), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != target) {
      if (it++ >= max_polls) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
    if (!ok) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  return __shfl(ok, 0, 64) != 0;
}

// Reader of tagged partial sums: t[j] for j = lane + 64 i < rank (i < 4), the
// sum over the S slices in slice order of the words of (tile j / 64, slice s),
// once all of them carry `tag`.  The words are read with device-scope loads
// (past the CU's own cache, which may hold an earlier launch's words), eight
// in flight at a time.  Bounded like wait_lowrank: a wait that gives up records
// it in the layer's error word and gives NaN.
__device__ __forceinline__ bool read_t_tagged(const float* part, int S, int rank, uint32_t tag, int lane, uint32_t max_polls,
                                              uint32_t* err, float (&tv)[4]) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const int ntj = (rank + 63) >> 6;
  const brsrc_t rp = make_rsrc(part, (uint32_t)ntj * (uint32_t)S * 512u);
  uint32_t it = 0;
  bool ok = false;
  for (;;) {
    bool mine = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = lane + 64 * i;
      float sum = 0.f;
      const uint32_t col = ((uint32_t)(j >> 6) * (uint32_t)S * 64u + (uint32_t)(j & 63)) * 8u;
      for (int s0 = 0; s0 < S; s0 += 8) {
        u32x2 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const bool live = j < rank && s0 + q < S;
          v[q] = __builtin_amdgcn_raw_buffer_load_b64(rp, live ? col + (uint32_t)(s0 + q) * 512u : kNoLoad, 0, 16);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (j < rank && s0 + q < S) {
            mine = mine && v[q].y == tag;
            sum += __uint_as_float(v[q].x);
          }
        }
      }
      tv[i] = sum;
    }
    if (__builtin_amdgcn_read_exec() == __ballot(mine)) {  // every lane's words are this launch's
      ok = true;
      break;
    }
    if (it++ >= max_polls) break;
    __builtin_amdgcn_s_sleep(4);
  }
  if (!ok) {
    if (lane == 0) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
#pragma unroll
    for (int i = 0; i < 4; ++i) tv[i] = lane + 64 * i < rank ? __builtin_nanf("") : 0.f;
  }
  return ok;
}

template <bool BF16>
__device__ __forceinline__ float dot2_act(uint32_t a, uint32_t b, float c) {
  if constexpr (BF16) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, a), __builtin_bit_cast(bf2, b), c, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
  }
}

// NT = threads of a prologue block.  A thread loads NL 16-byte pieces of the
// slice: 16 of fp16 / bf16 factors, 4 of int4 ones (1 or 4 in a 1024-thread
// block, NLX: the streaming kernel's choice per layer), so the slice has
// 2 (NT / 16) NL rows (16-bit) or 2 (NT / 4) NL rows (int4).
template <int MODE, int NT, int NLX = 0>
constexpr int lr_loads() { return NLX ? NLX : MODE == 0 ? 16 : NT == 1024 ? 1 : 4; }
template <int MODE, int NT, int NLX = 0>
constexpr int lr_slice_rows() { return 2 * (NT / (MODE == 0 ? 16 : 4)) * lr_loads<MODE, NT, NLX>(); }
static_assert(lr_slice_rows<0, 256>() == kLrSlice && lr_slice_rows<1, 256>() == kLrSlice, "256-thread slices");

template <int MODE, int MT, int NT = 256, int NLX = 0>
struct LrScratch {
  static constexpr int SL = lr_slice_rows<MODE, NT, NLX>();  // K rows of the slice
  static constexpr int NG = MODE == 0 ? NT / 64 : NT / 16;  // reduction groups left after the shuffles
  static constexpr int NSC = SL / 16 + 1;         // int4 scale rows a slice can touch (group >= 16)
  static constexpr int xs = 0;                                   // uint16 [MT][SL]
  static constexpr int sc = xs + MT * SL * 2;                    // float [NSC][64] (int4)
  static constexpr int red = sc + (MODE == 1 ? NSC * 64 * 4 : 16);  // float [NG][MT * 64]
  static constexpr int last = red + NG * MT * 64 * 4;            // int
  static constexpr int bytes = last + 16;
};

// LDS the block code needs (host side: sizes the decode kernel's dynamic LDS).
inline int lr_scratch_bytes(int mode, int mt, int nt = 256, int nl = 1) {
  if (nt == 1024) return mode == 0 ? LrScratch<0, 1, 1024>::bytes : nl == 4 ? LrScratch<1, 1, 1024, 4>::bytes : LrScratch<1, 1, 1024>::bytes;
  return mode == 0 ? (mt == 1 ? LrScratch<0, 1>::bytes : mt == 2 ? LrScratch<0, 2>::bytes : LrScratch<0, 4>::bytes)
                   : (mt == 1 ? LrScratch<1, 1>::bytes : mt == 2 ? LrScratch<1, 2>::bytes : LrScratch<1, 4>::bytes);
}

// One workgroup of the split prologue (NT working threads; a wider
// workgroup's threads past NT compute nothing that is kept): K slice s of
// LrScratch<MODE, MT, NT>::SL rows, column tile tj of ntj, activation tile tm;
// `smem` is LrScratch<MODE, MT, NT>::bytes of LDS.  EDIT: the activations may
// be raw (a.clamp, a.xscale apply); else they are edited already.
// Tagged partial sums (TAG, one activation row): instead of the arrival
// count, the last block's sum, the store of t and the published word, each
// block writes its 64 partial sums as 64-bit words (fp32 value, launch tag)
// that its readers load, check and add in slice order themselves -- one trip
// through memory instead of six.  The tag is the launch's epoch, or for a
// recorded launch its generation with the top bit set.
__device__ __forceinline__ uint32_t lr_tag(uint32_t epoch, uint32_t target) {
  return epoch ? epoch : (0x80000000u | target);
}

template <int MODE, int MT, bool BF16, bool EDIT, int NT = 256, bool TAG = false, int NLX = 0>
__device__ __forceinline__ void lr_split_block(const LrSplitArgs& a, int s, int tj, int tm, int ntj, uint8_t* smem) {
  using SC = LrScratch<MODE, MT, NT, NLX>;
  constexpr int SL = SC::SL;
  constexpr int NL = lr_loads<MODE, NT, NLX>();  // 16-byte loads per thread
  constexpr int JL = MODE == 0 ? 4 : 16;        // columns per thread
  constexpr int LG = 64 / JL;                   // threads per K pair row of the tile
  constexpr int PR = NT / LG;                   // K pair rows in flight per workgroup
  constexpr int NG = SC::NG;
  constexpr int XT = SL / 8;                    // threads staging one activation row of the slice
  static_assert(2 * PR * NL == SL, "the loads cover the slice");
  typedef uint16_t xrow_t[SL];
  typedef float redrow_t[MT * 64];
  xrow_t* xs = reinterpret_cast<xrow_t*>(smem + SC::xs);
  float* sc = reinterpret_cast<float*>(smem + SC::sc);
  redrow_t* red = reinterpret_cast<redrow_t*>(smem + SC::red);
  // an LDS-typed reference: smem reaches some callers as a generic pointer,
  // and a flat access would wait for every outstanding memory operation
  __attribute__((address_space(3))) int& s_last =
      *reinterpret_cast<__attribute__((address_space(3))) int*>(reinterpret_cast<uintptr_t>(smem + SC::last));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = s * SL, j0 = tj * 64, m0 = tm * MT;
  const int jg = tid % LG, pr = tid / LG;
  // the value this launch publishes, read before any work: the generation
  // cannot move while the launch's readers wait for it, and a publish that
  // comes late (after a reader gave up) then cannot run ahead of a later launch
  const uint32_t publish = a.flag != nullptr ? lr_target(a.flag, a.epoch) : 0u;

  // activations of the slice (zero past K and past M)
  const brsrc_t rx = make_rsrc(a.x, (uint32_t)a.M * (uint32_t)a.ldx * 2u);
  uint4 xv = make_uint4(0, 0, 0, 0);
  if (tid < MT * XT) {
    const int m = tid / XT, k = k0 + 8 * (tid % XT);
    const bool ok = m0 + m < a.M && k < a.ldx;
    xv = bload128(rx, ok ? ((uint32_t)(m0 + m) * (uint32_t)a.ldx + (uint32_t)k) * 2u : kNoLoad, 0);
  }
  uint4 xf = make_uint4(0, 0, 0, 0);
  if (EDIT && a.xscale && tid < MT * XT) {
    const int k = k0 + 8 * (tid % XT);
    xf = bload128(make_rsrc(a.xscale, (uint32_t)a.ldx * 2u), k < a.ldx ? (uint32_t)k * 2u : kNoLoad, 0);
  }
  // the slice of L
  const brsrc_t rl = make_rsrc(a.lk, MODE == 0 ? (uint32_t)a.Kl * (uint32_t)a.rpad * 2u : (uint32_t)a.Kl / 2u * (uint32_t)a.rpad);
  uint4 w[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {  // a wider workgroup's threads past NT load nothing
    const uint32_t p = (uint32_t)(k0 / 2 + pr + PR * i);
    w[i] = bload128(rl, tid >= NT ? kNoLoad
                        : MODE == 0 ? (p * (uint32_t)a.rpad + (uint32_t)(j0 + JL * jg)) * 4u
                                    : p * (uint32_t)a.rpad + (uint32_t)(j0 + JL * jg), 0);
  }
  // int4 scale rows of the slice, as fp32
  const int g0 = MODE == 1 ? k0 / a.group : 0;
  if constexpr (MODE == 1) {
    const int ng = (k0 + SL - 1) / a.group - g0 + 1;
    const brsrc_t rs = make_rsrc(a.ls, (uint32_t)((a.Kl + a.group - 1) / a.group) * (uint32_t)a.rpad * 2u);
    for (int i = tid; i < ng * 8; i += (int)blockDim.x) {
      const int row = i >> 3, part = i & 7;
      const uint4 v = bload128(rs, ((uint32_t)(g0 + row) * (uint32_t)a.rpad + (uint32_t)(j0 + 8 * part)) * 2u, 0);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[row * 64 + 8 * part + 2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[e] & 0xFFFFu));
        sc[row * 64 + 8 * part + 2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[e] >> 16));
      }
    }
  }
  if constexpr (EDIT) {
    if (a.clamp) xv = clamp_act8<BF16>(xv, a.cval);
    if (a.xscale) xv = scale_act8<BF16>(xv, xf);
  }
  if (tid < MT * XT) *reinterpret_cast<uint4*>(&xs[tid / XT][8 * (tid % XT)]) = xv;
  __syncthreads();

  float acc[MT][JL];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < JL; ++j) acc[m][j] = 0.f;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int pl = pr + PR * i;  // pair row within the slice
    if constexpr (MODE == 0) {
      const uint32_t wv[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint32_t xp = *reinterpret_cast<const uint32_t*>(&xs[m][2 * pl]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] = dot2_act<BF16>(wv[j], xp, acc[m][j]);
      }
    } else {
      const int k = k0 + 2 * pl;
      const float* s0 = &sc[(k / a.group - g0) * 64 + JL * jg];
      const float* s1 = &sc[((k + 1) / a.group - g0) * 64 + JL * jg];
      float x0[MT], x1[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint32_t xp = *reinterpret_cast<const uint32_t*>(&xs[m][2 * pl]);
        x0[m] = BF16 ? __uint_as_float(xp << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)(xp & 0xFFFFu));
        x1[m] = BF16 ? __uint_as_float(xp & 0xFFFF0000u) : (float)__builtin_bit_cast(_Float16, (uint16_t)(xp >> 16));
      }
      const uint32_t wv[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t byte = (wv[j >> 2] >> (8 * (j & 3))) & 0xFFu;
        const float v0 = (float)((int)(byte & 0xFu) - 8) * s0[j];
        const float v1 = (float)((int)(byte >> 4) - 8) * s1[j];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m][j] = __builtin_fmaf(v1, x1[m], __builtin_fmaf(v0, x0[m], acc[m][j]));
      }
    }
  }
  // lanes 16 and 32 apart hold other pair rows of the same columns
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < JL; ++j) {
      float v = acc[m][j];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      acc[m][j] = v;
    }
  if (lane < 16 && tid < NT) {  // a wider workgroup's threads past NT only keep the barriers
    const int grp = MODE == 0 ? wave : wave * 4 + (lane >> 2);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < JL; ++j) red[grp][m * 64 + JL * jg + j] = acc[m][j];
  }
  __syncthreads();
  float v = 0.f;
  const int o = tid;  // output m * 64 + column, for tid < MT * 64
  if (o < MT * 64) {
#pragma unroll
    for (int g = 0; g < NG; ++g) v += red[g][o];
  }
  if constexpr (TAG) {
    static_assert(MT == 1, "tagged partial sums of one activation row");
    if (o < 64) {
      const uint32_t tag = lr_tag(a.epoch, publish) ^ (a.withhold ? 0x40000000u : 0u);  // withheld: never matches
      uint64_t* dst = reinterpret_cast<uint64_t*>(a.part) + ((size_t)(tm * ntj + tj) * a.S + s) * 64 + o;
      __hip_atomic_store(dst, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  const int m = o >> 6, j = j0 + (o & 63);
  const bool store = o < MT * 64 && m0 + m < a.M && j < a.rank;
  const bool fused = a.flag != nullptr;
  float tv = v;
  if (a.S > 1) {
    const int tile = tm * ntj + tj;
    float* base = a.part + (size_t)tile * a.S * 256;
    if (o < MT * 64) store_dev(base + (size_t)s * 256 + o, v);
    wait_stores();
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(&a.cnt[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = old == (uint32_t)(a.S - 1) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    // last arrival: slices in order, eight loads in flight at a time
    if (o < MT * 64) {
      float sum = 0.f;
      for (int q0 = 0; q0 < a.S; q0 += 8) {
        float pv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) pv[q] = q0 + q < a.S ? load_dev(base + (size_t)(q0 + q) * 256 + o) : 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) sum += pv[q];
      }
      tv = sum;
    }
    if (tid == 0) __hip_atomic_store(&a.cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next forward
  }
  if (!fused) {
    if (store) a.t[(size_t)(m0 + m) * a.rank + j] = tv;
    return;
  }
  // inside the decode kernel: t through the coherent path, then count the
  // tile; the last tile publishes this launch's epoch or generation
  if (store) store_dev(a.t + (size_t)(m0 + m) * a.rank + j, tv);
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint32_t)(a.ntiles - 1)) {
      __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next forward
      if (!a.withhold) __hip_atomic_store(lr_word(a.flag, a.epoch), publish, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Activation rows per prologue tile for a batch of M.
inline int lowrank_tile_m(int M) { return M == 1 ? 1 : M == 2 ? 2 : 4; }

// Arguments of the split prologue for a forward (flag NULL: a kernel of its own).
LrSplitArgs lowrank_split_args(const Layer& L, int M, const void* x);

}  // namespace cl
