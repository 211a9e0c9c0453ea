// unpack.h -- device functions that turn packed chunks into fp16 weight pairs.
//
// One lane owns one row of a 64-row tile.  Every function here returns the
// dequantised weights of one chunk of that row as `uint32_t` words, each the
// bit pattern of two fp16 values (low half = even k, high half = odd k), so
// that the forward can multiply them with pairs of activations and the debug
// kernel can store them.  The forward, the debug kernel and the prefill
// dequantiser all call these same functions.
//
// LUT lookups go through tables in LDS laid out "lane-interleaved": entry e of
// lane l is the dword at byte address e*256 + l*4.  The 64 lanes of a
// wavefront then always hit 64 distinct banks (dword l of each 256-byte row),
// whatever codes they look up, and the address is built with one v_perm_b32:
// the code (or code pair) byte goes into address byte 1, the lane offset
// l*4 stays in byte 0.  This needs the table to start at LDS address 0, so
// every kernel that uses these tables declares exactly one __shared__ array.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cl {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t perm(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// LDS reads at a byte address inside the kernel's LDS array `lds`.  The array
// is the kernel's only LDS object, so it starts at address 0 and byte_addr is
// also its absolute LDS address (the v_perm address tricks rely on that).
// Indexing through `lds` keeps the table stores visibly live to the compiler.
__device__ __forceinline__ uint32_t lds_u32(const uint32_t* lds, uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(lds) + byte_addr);
}
__device__ __forceinline__ uint32_t lds_u16(const uint32_t* lds, uint32_t byte_addr) {
  return *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(lds) + byte_addr);
}
__device__ __forceinline__ uint2 lds_u64(const uint32_t* lds, uint32_t byte_addr) {
  return *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(lds) + byte_addr);
}

// Device-scope (all XCDs) relaxed atomic store / load of one float, and a wait
// until this wave's stores have completed (written through to the coherent level).
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), expcnt(7), lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Raw buffer loads: a 32-bit per-lane byte offset plus a uniform one, and a
// hardware range check against the buffer size (loads past it return zero).
typedef __amdgpu_buffer_rsrc_t brsrc_t;
typedef uint32_t bu32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ brsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload128(brsrc_t r, uint32_t voff, uint32_t soff) {
  const bu32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Loads of data read once (the code stream), with the non-temporal cache
// policy: on a long stream they reach a higher rate (6.1 vs 5.5 TB/s measured
// on a 105 MB read).
__device__ __forceinline__ uint4 bload128_nt(brsrc_t r, uint32_t voff, uint32_t soff) {
  const bu32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 bload64_nt(brsrc_t r, uint32_t voff, uint32_t soff) {
  typedef uint32_t bu32x2 __attribute__((ext_vector_type(2)));
  const bu32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 2);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint2 bload64(brsrc_t r, uint32_t voff, uint32_t soff) {
  typedef uint32_t bu32x2 __attribute__((ext_vector_type(2)));
  const bu32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t bload32(brsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bload16(brsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bload8(brsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}
// A buffer offset past any buffer this library makes (all are below 2 GiB):
// the load returns zero.
constexpr uint32_t kNoLoad = 0x80000000u;

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// address byte 1 <- byte `i` of `src`; bytes 0, 2, 3 from `lanebase`
template <int I>
__device__ __forceinline__ uint32_t addr_from_byte(uint32_t src, uint32_t lanebase) {
  return perm(src, lanebase, 0x03020000u | ((4u + I) << 8));
}

// ---------------------------------------------------------------------------
// 3-bit LUT: pair table.  Entry (a | b << 3) holds fp16 lut[a] (low) and
// lut[b] (high): one lookup dequantises two consecutive weights.  The packed
// byte j reads 4 * p_j for the first four pairs; the fifth pair's three 2-bit
// pieces (bits 0-1 of bytes 0..2) are gathered by one 24-bit multiply into
// byte 2 as 4 * p_4 (the partial products do not overlap).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lut3_p4x4(uint32_t w) {  // byte 2 = 4 * p_4
  return __umul24(w & 0x00030303u, 0x41040u);
}

// Lane-interleaved table (entry e of lane l at e*256 + 4*l): entry index in
// address byte 1.  `ebias` is ORed into every entry byte (selects one of
// several stacked tables: 64 * g for table g).
__device__ __forceinline__ void lut3_word(const uint32_t* lds, uint32_t w, uint32_t lanebase, uint32_t out[5],
                                         uint32_t ebias = 0) {
  const uint32_t m = ((w >> 2) & 0x3F3F3F3Fu) | (ebias * 0x01010101u);
  const uint32_t p4 = (lut3_p4x4(w) >> 2) | (ebias << 16);  // byte 2 = p_4
  out[0] = lds_u32(lds, addr_from_byte<0>(m, lanebase));
  out[1] = lds_u32(lds, addr_from_byte<1>(m, lanebase));
  out[2] = lds_u32(lds, addr_from_byte<2>(m, lanebase));
  out[3] = lds_u32(lds, addr_from_byte<3>(m, lanebase));
  out[4] = lds_u32(lds, addr_from_byte<2>(p4, lanebase));
}

// 3-bit LUT dequantisation without table lookups: the 8 values of a row in the
// MFMA input type, as byte tables for v_perm (low bytes of values 0..3 / 4..7,
// high bytes of values 0..3 / 4..7), held in registers.
struct Lut3Bytes {
  uint32_t l0, l1, h0, h1;
};

// The row's 8 fp16 LUT values (one 16-byte load) as byte tables, rounded to
// nearest-even bf16 first when the MFMAs run in bf16.
template <bool BF16>
__device__ __forceinline__ Lut3Bytes lut3_bytes(uint4 lv) {
  const uint32_t lw[4] = {lv.x, lv.y, lv.z, lv.w};
  uint32_t v16[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t h = (lw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    v16[e] = BF16 ? (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(float)__builtin_bit_cast(_Float16, (uint16_t)h)) : h;
  }
  Lut3Bytes T;
  T.l0 = (v16[0] & 0xFF) | (v16[1] & 0xFF) << 8 | (v16[2] & 0xFF) << 16 | (v16[3] & 0xFF) << 24;
  T.l1 = (v16[4] & 0xFF) | (v16[5] & 0xFF) << 8 | (v16[6] & 0xFF) << 16 | (v16[7] & 0xFF) << 24;
  T.h0 = (v16[0] >> 8) | (v16[1] >> 8) << 8 | (v16[2] >> 8) << 16 | (v16[3] >> 8) << 24;
  T.h1 = (v16[4] >> 8) | (v16[5] >> 8) << 8 | (v16[6] >> 8) << 16 | (v16[7] >> 8) << 24;
  return T;
}

// Ten 3-bit codes of a device word (byte j < 4: bits 2..4 code 2j, bits 5..7
// code 2j + 1; the fifth pair from the low two bits of bytes 0..2) into five
// pairs of values: each byte of a selector word picks one value's low (or
// high) byte from the row's tables (about 2.4 vector instructions per weight).
__device__ __forceinline__ void lut3_word_perm(uint32_t w, const Lut3Bytes& T, uint32_t out[5]) {
  const uint32_t ev = (w >> 2) & 0x07070707u, od = (w >> 5) & 0x07070707u;
  const uint32_t loE = perm(T.l1, T.l0, ev), hiE = perm(T.h1, T.h0, ev);
  const uint32_t loO = perm(T.l1, T.l0, od), hiO = perm(T.h1, T.h0, od);
  const uint32_t e01 = perm(hiE, loE, 0x05010400u), e23 = perm(hiE, loE, 0x07030602u);
  const uint32_t o01 = perm(hiO, loO, 0x05010400u), o23 = perm(hiO, loO, 0x07030602u);
  out[0] = perm(o01, e01, 0x05040100u);
  out[1] = perm(o01, e01, 0x07060302u);
  out[2] = perm(o23, e23, 0x05040100u);
  out[3] = perm(o23, e23, 0x07060302u);
  const uint32_t p = lut3_p4x4(w) >> 18;  // code 8 in bits 0..2, code 9 in bits 3..5
  const uint32_t s = (p & 7u) | ((p & 0x38u) << 5);
  const uint32_t lo = perm(T.l1, T.l0, s), hi = perm(T.h1, T.h0, s);
  out[4] = perm(hi, lo, 0x05010400u);
}

// Row table (entry e of the row at rowbase + 4*e, rowbase a multiple of 256):
// the byte 4 * p goes straight into address byte 0.
__device__ __forceinline__ void lut3_word_row(const uint32_t* lds, uint32_t w, uint32_t rowbase, uint32_t out[5]) {
  const uint32_t m = w & 0xFCFCFCFCu;
  const uint32_t p4 = lut3_p4x4(w);
  out[0] = lds_u32(lds, perm(m, rowbase, 0x03020104u));
  out[1] = lds_u32(lds, perm(m, rowbase, 0x03020105u));
  out[2] = lds_u32(lds, perm(m, rowbase, 0x03020106u));
  out[3] = lds_u32(lds, perm(m, rowbase, 0x03020107u));
  out[4] = lds_u32(lds, perm(p4, rowbase, 0x03020106u));
}

// 4-bit LUT, row pair table of 256 entries (entry p = lut[p & 15] | lut[p >> 4]
// << 16) at rowbase, a multiple of 1024 below 64 KiB.  The packed byte holds
// the pair rotated left by 2: its bits 2..7 are address byte 0 (4 * (p mod 64)),
// its bits 0..1 with the row base form address byte 1.
__device__ __forceinline__ void lut4_pair_row(const uint32_t* lds, uint32_t w, uint32_t rowbase, uint32_t out[4]) {
  const uint32_t lo = w & 0xFCFCFCFCu;
  const uint32_t hi = (w & 0x03030303u) | ((rowbase >> 8) * 0x01010101u);
  out[0] = lds_u32(lds, perm(hi, lo, 0x0C0C0400u));
  out[1] = lds_u32(lds, perm(hi, lo, 0x0C0C0501u));
  out[2] = lds_u32(lds, perm(hi, lo, 0x0C0C0602u));
  out[3] = lds_u32(lds, perm(hi, lo, 0x0C0C0703u));
}

// The canonical nibble order of a packed LUT4 word (each byte rotated back right by 2).
__device__ __forceinline__ uint32_t lut4_canon(uint32_t w) {
  return ((w >> 2) & 0x3F3F3F3Fu) | ((w << 6) & 0xC0C0C0C0u);
}

// ---------------------------------------------------------------------------
// 4-bit LUT: single-code table, entry c = fp16 lut[c] in the low half.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lut4_word(const uint32_t* lds, uint32_t w, uint32_t lanebase, uint32_t out[4],
                                         uint32_t ebias = 0) {
  w = lut4_canon(w);
  const uint32_t ev = (w & 0x0F0F0F0Fu) | (ebias * 0x01010101u);         // codes of even k, one per byte
  const uint32_t od = ((w >> 4) & 0x0F0F0F0Fu) | (ebias * 0x01010101u);  // codes of odd k
  uint32_t lo[4], hi[4];
  lo[0] = lds_u16(lds, addr_from_byte<0>(ev, lanebase));
  hi[0] = lds_u16(lds, addr_from_byte<0>(od, lanebase));
  lo[1] = lds_u16(lds, addr_from_byte<1>(ev, lanebase));
  hi[1] = lds_u16(lds, addr_from_byte<1>(od, lanebase));
  lo[2] = lds_u16(lds, addr_from_byte<2>(ev, lanebase));
  hi[2] = lds_u16(lds, addr_from_byte<2>(od, lanebase));
  lo[3] = lds_u16(lds, addr_from_byte<3>(ev, lanebase));
  hi[3] = lds_u16(lds, addr_from_byte<3>(od, lanebase));
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = perm(hi[j], lo[j], 0x05040100u);
}

// ---------------------------------------------------------------------------
// Integers to fp16 without a convert: 0x6400 | u is the fp16 value 1024 + u
// for 0 <= u < 1024, so subtracting the bias (1024 + offset) gives q exactly.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t int4_pair(uint32_t w, int shift) {
  const uint32_t b = ((w >> shift) & 0x000F000Fu) | 0x64006400u;  // 1024 + u, u = q + 8
  const half2_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  return as_u32(as_h2(b) - bias);
}

__device__ __forceinline__ void int4_word(uint32_t w, uint32_t out[4]) {
  out[0] = int4_pair(w, 0);
  out[1] = int4_pair(w, 4);
  out[2] = int4_pair(w, 8);
  out[3] = int4_pair(w, 12);
}

__device__ __forceinline__ void int8_word(uint32_t w, uint32_t out[2]) {
  const half2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};      // 1024 + 128
  out[0] = as_u32(as_h2(perm(0x64646464u, w, 0x04010400u)) - bias);  // bytes 0, 1
  out[1] = as_u32(as_h2(perm(0x64646464u, w, 0x04030402u)) - bias);  // bytes 2, 3
}

// 2:4 group: kept pair Q = (v0, v1) and the selector entry for its meta nibble
// expand into the four weights of the group (two fp16 pairs); positions not
// kept read selector value 12, which v_perm turns into a zero byte.
__device__ __forceinline__ void int4_24_group(const uint32_t* lds, uint32_t vw, int g4, uint32_t meta_word, int g8,
                                              uint32_t seltab_base, uint32_t out[2]) {
  const uint32_t q = int4_pair(vw, 4 * g4);
  const uint32_t nib = (meta_word >> (4 * g8)) & 0xFu;
  const uint2 sel = lds_u64(lds, seltab_base + nib * 8u);
  out[0] = perm(q, q, sel.x);
  out[1] = perm(q, q, sel.y);
}

// Selector table of the 2:4 expansion (16 entries x 2 dwords); nibble = i0 | i1 << 2.
__device__ __forceinline__ uint2 seltab_2_4_entry(uint32_t nib) {
  const uint32_t i0 = nib & 3u, i1 = nib >> 2;
  uint32_t bytes[4];
#pragma unroll
  for (uint32_t p = 0; p < 4; ++p) {
    // selector bytes of fp16 position p: Q bytes (0,1) for the first kept,
    // (2,3) for the second, (12,12) -> zero when p is dropped
    bytes[p] = (p == i0) ? 0x0100u : (p == i1 && i1 != i0) ? 0x0302u : 0x0C0Cu;
  }
  return make_uint2(bytes[0] | (bytes[1] << 16), bytes[2] | (bytes[3] << 16));
}

// Nibble selector of the bitmap expansion: byte p of the entry is the rank of
// weight p among the kept weights of the nibble, or 12 (zero) if p is dropped.
__device__ __forceinline__ uint32_t bitmap_sel_entry(uint32_t nib) {
  uint32_t r = 0, sel = 0;
#pragma unroll
  for (uint32_t p = 0; p < 4; ++p) {
    const bool kept = (nib >> p) & 1u;
    sel |= (kept ? r : 12u) << (8 * p);
    r += kept;
  }
  return sel;
}

// Four signed int8 weights (dropped ones already zero) to two fp16 pairs.
__device__ __forceinline__ void int8x4_signed(uint32_t d4, uint32_t out[2]) {
  int8_word(d4 ^ 0x80808080u, out);
}


// ---------------------------------------------------------------------------
// Per-kind chunk dequantisation (shared by the forward, the debug kernel and
// the prefill tile loader).
// ---------------------------------------------------------------------------
enum Kind { K_LUT3 = 0, K_LUT4, K_INT4, K_INT4_24, K_INT8, K_INT8_BM };

template <int KIND>
constexpr bool is_int_kind() { return KIND == K_INT4 || KIND == K_INT4_24 || KIND == K_INT8 || KIND == K_INT8_BM; }

// Bitmap expansion: 16 nibble selectors, then one staging slot per dense lane
// of 35 dwords (odd stride: the 64 lanes fall in distinct banks); a slot holds
// the <= 128 kept bytes of one chunk plus alignment slack.
constexpr int kBmSlot = 35;
constexpr int kBmSelDwords = 16;

template <int KIND>
struct KindTraits;
template <> struct KindTraits<K_LUT3> { static constexpr int span = 40, pairs = 20, tab_dwords = 64 * 64; };
template <> struct KindTraits<K_LUT4> { static constexpr int span = 32, pairs = 16, tab_dwords = 16 * 64; };
template <> struct KindTraits<K_INT4> { static constexpr int span = 32, pairs = 16, tab_dwords = 0; };
template <> struct KindTraits<K_INT4_24> { static constexpr int span = 64, pairs = 32, tab_dwords = 32; };
template <> struct KindTraits<K_INT8> { static constexpr int span = 16, pairs = 8, tab_dwords = 0; };
template <> struct KindTraits<K_INT8_BM> { static constexpr int span = 128, pairs = 64, tab_dwords = kBmSelDwords + 4 * 64 * kBmSlot; };

// Dequantise one chunk of this lane's row into fp16 pairs wp[j] = (k = 2j, 2j+1).
//   w          the 16-byte chunk of the dense stream (bitmap: the keep bits)
//   mw         2:4 metadata (x, y) of the chunk
//   lanebase   lane * 4 (LUT tables), slot_base: byte address of the lane's
//              staged kept values (bitmap), already offset to the first one
//   ROWTAB     LUT tables are per-row tables at `lanebase` (rowbase) instead of
//              lane-interleaved tables
//   ebias      lane-interleaved tables only: ORed into the entry index (stacked tables)
template <int KIND, bool ROWTAB = false>
__device__ __forceinline__ void chunk_pairs(const uint32_t* lds, uint4 w, uint4 mw, uint32_t lanebase, uint32_t slot_base,
                                            uint32_t (&wp)[KindTraits<KIND>::pairs], uint32_t ebias = 0) {
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  if constexpr (KIND == K_LUT3 && ROWTAB) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lut3_word_row(lds, ww[i], lanebase, &wp[5 * i]);
  } else if constexpr (KIND == K_LUT4 && ROWTAB) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lut4_pair_row(lds, ww[i], lanebase, &wp[4 * i]);
  } else if constexpr (KIND == K_LUT3) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lut3_word(lds, ww[i], lanebase, &wp[5 * i], ebias);
  } else if constexpr (KIND == K_LUT4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lut4_word(lds, ww[i], lanebase, &wp[4 * i], ebias);
  } else if constexpr (KIND == K_INT4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) int4_word(ww[i], &wp[4 * i]);
  } else if constexpr (KIND == K_INT4_24) {
    const uint32_t mm[2] = {mw.x, mw.y};
#pragma unroll
    for (int g = 0; g < 16; ++g) int4_24_group(lds, ww[g / 4], g % 4, mm[g / 8], g % 8, 0u, &wp[2 * g]);
  } else if constexpr (KIND == K_INT8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) int8_word(ww[i], &wp[2 * i]);
  } else {
    uint32_t off = slot_base;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t nib = (ww[i] >> (4 * t)) & 0xFu;
        const uint32_t lo = lds_u32(lds, off & ~3u), hi = lds_u32(lds, (off & ~3u) + 4u);
        const uint32_t win = __builtin_amdgcn_alignbyte(hi, lo, off & 3u);
        const uint32_t d4 = perm(0u, win, lds_u32(lds, nib * 4u));
        int8x4_signed(d4, &wp[16 * i + 2 * t]);
        off += __builtin_popcount(nib);
      }
    }
  }
}

// LDS tables of a 64-row tile, built by `nthreads` threads (>= 64, a multiple of 64):
// LUT pair / single tables at address 0, or the selector tables.
template <int KIND>
__device__ __forceinline__ void build_tables(uint32_t* smem, const uint16_t* table, int tile, int tid, int nthreads) {
  const int lane = tid & 63, grp = tid >> 6, ngrp = nthreads >> 6;
  const int n = tile * 64 + lane;
  if constexpr (KIND == K_LUT3) {
    const uint4 lv = reinterpret_cast<const uint4*>(table)[n];
    const uint32_t lw[4] = {lv.x, lv.y, lv.z, lv.w};
    for (int i = grp; i < 64; i += ngrp) {
      const int ca = i & 7, cb = i >> 3;
      const uint32_t va = (lw[ca >> 1] >> (16 * (ca & 1))) & 0xFFFFu;
      const uint32_t vb = (lw[cb >> 1] >> (16 * (cb & 1))) & 0xFFFFu;
      smem[i * 64 + lane] = va | (vb << 16);
    }
  } else if constexpr (KIND == K_LUT4) {
    const uint4 l0 = reinterpret_cast<const uint4*>(table)[2 * n];
    const uint4 l1 = reinterpret_cast<const uint4*>(table)[2 * n + 1];
    const uint32_t lw[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
    for (int c = grp; c < 16; c += ngrp) smem[c * 64 + lane] = (lw[c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
  } else if constexpr (KIND == K_INT4_24) {
    if (tid < 16) {
      const uint2 e = seltab_2_4_entry((uint32_t)tid);
      smem[2 * tid] = e.x;
      smem[2 * tid + 1] = e.y;
    }
  } else if constexpr (KIND == K_INT8_BM) {
    if (tid < 16) smem[tid] = bitmap_sel_entry((uint32_t)tid);
  }
}

// Per-row LUT tables of `nrows` consecutive rows starting at row0 (LUT3: 64
// pair entries, row q at byte q*256; LUT4: 256 pair entries, row q at byte
// q*1024); the 2:4 and bitmap selector tables at address 0 as for the tile tables.
template <int KIND>
constexpr int row_table_bytes() { return KIND == K_LUT4 ? 1024 : 256; }
template <int KIND>
__device__ __forceinline__ void build_row_tables(uint32_t* smem, const uint16_t* table, int row0, int nrows, int tid,
                                                 int nthreads) {
  if constexpr (KIND == K_LUT3) {
    for (int i = tid; i < nrows * 64; i += nthreads) {
      const int q = i >> 6, e = i & 63, ca = e & 7, cb = e >> 3;
      const uint16_t* lt = table + (size_t)(row0 + q) * 8;
      smem[q * 64 + e] = (uint32_t)lt[ca] | ((uint32_t)lt[cb] << 16);
    }
  } else if constexpr (KIND == K_LUT4) {
    for (int i = tid; i < nrows * 256; i += nthreads) {
      const int q = i >> 8, e = i & 255;
      const uint16_t* lt = table + (size_t)(row0 + q) * 16;
      smem[q * 256 + e] = (uint32_t)lt[e & 15] | ((uint32_t)lt[e >> 4] << 16);
    }
  } else {
    build_tables<KIND>(smem, table, 0, tid, nthreads < 64 ? 64 : nthreads);
  }
}

}  // namespace cl
